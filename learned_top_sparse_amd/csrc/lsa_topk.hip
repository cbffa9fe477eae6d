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
#include <algorithm>
#include <atomic>
#include <climits>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_idx_tiles.h"
#include "lsa_select.h"

namespace lsa {

namespace {


__device__ __forceinline__ unsigned okey(int s) { return (unsigned)s ^ 0x80000000u; }

// Among positions [0, n) accepted by pred (payload = score), find the need-th best
// score by 8-bit radix passes on the order-preserving key.  Returns T (as key) and
// sets *need_eq to how many entries equal to T are selected.  All threads call.
template <int NT, int V, typename Pred>
__device__ __forceinline__ unsigned radix_select32(int n, int need, int* h256, int* scan_tmp, int* sh,
                                                   Pred pred, int* need_eq, int shift0 = 24, unsigned pref0 = 0u,
                                                   unsigned pmask0 = 0u) {
  unsigned pref = pref0, pmask = pmask0;
  for (int shift = shift0; shift >= 0; shift -= 8) {
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

// ---------------------------------------------------------------------------------
// One query row as seen by the selection: candidate slots [0, n_slots), their
// scores in global memory, and (two-stage mode) the kept-block table in LDS.  The
// written list holds key_of(slot): the key (two-stage: through the kept blocks), or
// with paged caches (pt set) the key's pool row.
template <bool KEPT>
struct RowView {
  const int32_t* srow;
  const int* kept_s;  // KEPT: block table in LDS
  int n_slots, p, bs;
  bool vec;           // 16-byte aligned row: vector loads
  const int32_t* pt = nullptr;  // paged caches: the row's page table (page ids clamped to n_pages)
  int plog2 = 0, n_pages = 0;
  // KEPT: the kept-table index of slot s is s / bs, taken without a division: a shift
  // when bs is a power of two, else the high half of s * (floor(2^32 / bs) + 1), which
  // is exact for 0 <= s < 2^16 (slots are fewer than 256 * 128)
  int bs_log2 = -1;
  unsigned bs_magic = 0;

  __device__ __forceinline__ void set_block_size(int b) {
    bs = b;
    bs_log2 = (b & (b - 1)) == 0 ? __builtin_ctz((unsigned)b) : -1;
    bs_magic = bs_log2 >= 0 ? 0u : (unsigned)(0xFFFFFFFFu / (unsigned)b) + 1u;
  }
  __device__ __forceinline__ int blk_of(int s) const {
    return bs_log2 >= 0 ? (s >> bs_log2) : (int)__umulhi((unsigned)s, bs_magic);
  }
  __device__ __forceinline__ int key_of(int s) const {
    int key = s;
    if constexpr (KEPT) {
      const int bi = blk_of(s);
      key = kept_s[bi] * bs + (s - bi * bs);
    }
    if (pt == nullptr) return key;
    return (min(max(pt[key >> plog2], 0), n_pages - 1) << plog2) | (key & ((1 << plog2) - 1));
  }
  __device__ __forceinline__ bool valid(int s) const {
    if (s >= n_slots) return false;
    if constexpr (KEPT) {
      const int bi = blk_of(s);
      const int blk = kept_s[bi];
      return blk >= 0 && blk * bs + (s - bi * bs) <= p;
    } else {
      return true;
    }
  }
  // scores of slots s0..s0+3 (s0 % 4 == 0) and a 4-bit candidate mask
  __device__ __forceinline__ unsigned load4(int s0, int (&sc)[4]) const {
    if (vec && s0 + 3 < n_slots) {
      const v4i x = *(const v4i*)(srow + s0);
      sc[0] = x[0]; sc[1] = x[1]; sc[2] = x[2]; sc[3] = x[3];
      if constexpr (!KEPT) return 0xFu;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[c] = (s0 + c < n_slots) ? srow[s0 + c] : 0;
    }
    unsigned m = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) m |= (valid(s0 + c) ? 1u : 0u) << c;
    return m;
  }
};

// Ordered emission of one pass of 4*V*NT positions starting at `base`: thread t
// holds positions base + 4*(v*NT + t) + c (c < 4) with selection bits m[v] and
// payloads pl[v][c]; emit(rank, pos, payload) gets every selected position with its
// rank in position order, starting at `running`.  wcnt: LDS int[V * NT/64].  One
// barrier; all threads call; returns running + count.
template <int NT, int V, typename P, typename Emit>
__device__ __forceinline__ int ordered_emit4(int base, const unsigned (&m)[V], const P (&pl)[V][4], int* wc,
                                             int running, Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long bal[V][4];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) bal[v][c] = __ballot((m[v] >> c) & 1u);
  if (lane == 0) {
#pragma unroll
    for (int v = 0; v < V; ++v)
      wc[v * NW + wave] = __popcll(bal[v][0]) + __popcll(bal[v][1]) + __popcll(bal[v][2]) + __popcll(bal[v][3]);
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
    if (m[v]) {
      int r = off + pre;
#pragma unroll
      for (int c = 0; c < 4; ++c) r += lanes_below(bal[v][c]);
      const int pos4 = base + 4 * (v * NT + (int)threadIdx.x);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((m[v] >> c) & 1u) emit(r++, pos4 + c, pl[v][c]);
    }
    off += tot;
  }
  return off;
}

// Ordered compaction over positions [lo, hi) (lo % 4 == 0) taken four at a time:
// f4(pos4, payload[4]) returns a 4-bit selection mask; emit(rank, pos, payload) gets
// each selected position with its rank in position order, starting at `running`.
// One barrier per 4*V*NT positions.  All threads call; returns running + count.
template <int NT, int V, typename F4, typename Emit>
__device__ __forceinline__ int ordered_compact4(int lo, int hi, int* wcnt, int running, F4 f4, Emit emit) {
  constexpr int NW = NT / 64;
  int parity = 0;
  for (int base = lo; base < hi; base += 4 * V * NT) {
    unsigned m[V];
    int pl[V][4];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int pos4 = base + 4 * (v * NT + (int)threadIdx.x);
      m[v] = 0;
      if (pos4 < hi) {
        m[v] = f4(pos4, pl[v]);
        const int left = hi - pos4;
        if (left < 4) m[v] &= (1u << left) - 1u;
      }
    }
    running = ordered_emit4<NT, V>(base, m, pl, wcnt + parity * V * NW, running, emit);
    parity ^= 1;
  }
  __syncthreads();
  return running;
}

// Coarse-bin histogram of the candidates in slots [lo, hi) into LDS `hist`.
template <int NT, int V, bool KEPT>
__device__ __forceinline__ void row_histogram(const RowView<KEPT> rv, int lo, int hi, int* hist) {
  for (int base = lo; base < hi; base += 4 * V * NT) {
    int sc[V][4];
    unsigned m[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int s0 = base + 4 * (v * NT + (int)threadIdx.x);
      m[v] = 0;
      if (s0 < hi) {
        m[v] = rv.load4(s0, sc[v]);
        const int left = hi - s0;
        if (left < 4) m[v] &= (1u << left) - 1u;
      }
    }
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((m[v] >> c) & 1u) atomicAdd(&hist[coarse_bin(sc[v][c])], 1);
  }
}

// Steps 4-5 once the entries of bins >= b* sit in slot order in the LDS list
// (lslot, lval; Lc entries): exact threshold inside b*, then the output row.
// Bits shared by the (score, -slot) keys of every entry of coarse bin b: a bin is a
// power-of-two aligned score range, so its scores agree above the range's width
// (in the order-preserving unsigned form).  Returns the mask of those key bits and
// sets *pref to their value.
__device__ __forceinline__ unsigned long long bin_key_prefix(int b, unsigned long long* pref) {
  const unsigned lo = okey(bin_floor(b));
  const unsigned hi = b >= 7295 ? 0xFFFFFFFFu : okey(bin_floor(b + 1)) - 1u;
  const unsigned d = lo ^ hi;
  const unsigned long long m = d == 0u ? 0xFFFFFFFF00000000ull : ~((2ull << (63 - __clzll((long long)d << 32))) - 1ull);
  *pref = ((unsigned long long)lo << 32) & m;
  return m;
}

// The need-th largest of n <= 64*KPW 64-bit keys (1 <= need <= n), exactly, by one
// wave holding KPW keys per lane in registers: a radix select over the bits where
// the keys differ, 8 at a time from the highest, with its own 256-bucket histogram
// in LDS (a wave's LDS operations take effect in order, so no barrier is needed),
// stopping early once every key left in the chosen bucket is taken (the cutoff is
// then the smallest of them).  key(i) gives key i (and may be called, its value
// unused, for any i < 64*KPW); every key agrees with pref0 on the bits of pmask0 (0,
// 0: nothing known), which the passes skip.
template <int KPW, typename Key>
__device__ __forceinline__ unsigned long long wave_select_kth(int n, int need, Key key, int* h256,
                                                              unsigned long long pref0 = 0ull,
                                                              unsigned long long pmask0 = 0ull) {
  const int lane = threadIdx.x & 63;
  auto wave_min = [&](unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long w = (unsigned long long)__shfl_xor((long long)v, o);
      v = w < v ? w : v;
    }
    return v;
  };
  unsigned long long kv[KPW];  // read unconditionally (key(i) must be readable for i < 64*KPW)
#pragma unroll
  for (int j = 0; j < KPW; ++j) kv[j] = key(lane + 64 * j);
  // the radix starts at the byte holding the highest bit not fixed by pmask0
  const int hb = pmask0 == ~0ull ? -1 : 63 - __clzll((long long)~pmask0);
  if (hb < 0) return pref0;
  int shift = (hb / 8) * 8;
  unsigned long long pmask = shift + 8 >= 64 ? 0ull : ~((1ull << (shift + 8)) - 1ull);
  unsigned long long pref = pref0 & pmask;  // pmask0 is a prefix mask, so pmask is inside it
  for (; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) h256[lane + 64 * j] = 0;
#pragma unroll
    for (int j = 0; j < KPW; ++j)
      if (lane + 64 * j < n && (kv[j] & pmask) == pref) atomicAdd(&h256[(int)((kv[j] >> shift) & 255ull)], 1);
    // lane l holds buckets 255-4l .. 252-4l (highest first); inclusive scan over lanes
    int c[4], lsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = h256[255 - 4 * lane - j];
      lsum += c[j];
    }
    int incl = lsum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int excl = incl - lsum;
    const unsigned long long hit = __ballot(excl < need && incl >= need);
    const int src = (int)__ffsll((long long)hit) - 1;
    int d = 0, before = 0, in_bucket = 0;
    if (lane == src) {
      int acc = excl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (acc + c[j] >= need) {
          d = 255 - 4 * lane - j;
          before = acc;
          in_bucket = c[j];
          break;
        }
        acc += c[j];
      }
    }
    d = __shfl(d, src);
    before = __shfl(before, src);
    in_bucket = __shfl(in_bucket, src);
    need -= before;
    pref |= (unsigned long long)d << shift;
    pmask |= 255ull << shift;
    if (in_bucket == need) {  // every key left is taken
      unsigned long long mn = ~0ull;
#pragma unroll
      for (int j = 0; j < KPW; ++j)
        if (lane + 64 * j < n && (kv[j] & pmask) == pref && kv[j] < mn) mn = kv[j];
      return wave_min(mn);
    }
  }
  return pref;
}

template <int NT, bool KEPT>
__device__ __forceinline__ void finish_from_list(const RowView<KEPT> rv, int Lc, int* lslot, int* lval, int bstar,
                                                 int above, int k, int* wcnt, int* h256, int* scan_tmp, int* sh,
                                                 int32_t* out) {
  // bits shared by every entry of b*: the radix starts at the byte of the highest differing bit
  unsigned mx = 0u, mn = 0xFFFFFFFFu;
  for (int e = threadIdx.x; e < Lc; e += NT) {
    const int sc = lval[e];
    if (coarse_bin(sc) == bstar) {
      const unsigned u = okey(sc);
      mx = u > mx ? u : mx;
      mn = u < mn ? u : mn;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    mx = max(mx, (unsigned)__shfl_xor((int)mx, o));
    mn = min(mn, (unsigned)__shfl_xor((int)mn, o));
  }
  if (threadIdx.x == 0) {
    sh[2] = 0;
    sh[3] = -1;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    atomicMax((unsigned*)&sh[2], mx);
    atomicMin((unsigned*)&sh[3], mn);
  }
  __syncthreads();
  mx = (unsigned)sh[2];
  mn = (unsigned)sh[3];
  __syncthreads();
  int need_eq;
  unsigned T;
  if (mx == mn) {  // every entry of b* has the same score
    T = mx;
    need_eq = k - above;
  } else {
    const int hb = 31 - __clz((int)(mx ^ mn));
    const int shift0 = (hb / 8) * 8;
    const unsigned pmask0 = shift0 + 8 >= 32 ? 0u : ~((1u << (shift0 + 8)) - 1u);
    T = radix_select32<NT, 4>(
        Lc, k - above, h256, scan_tmp, sh,
        [&](int e, int& sc) {
          sc = lval[e];
          return coarse_bin(sc) == bstar;
        },
        &need_eq, shift0, mx & pmask0, pmask0);
  }
  ordered_compact<NT, 4>(
      Lc, wcnt, [&](int e, int&) { return okey(lval[e]) == T; },
      [&](int r, int e, int) {
        if (r >= need_eq) lslot[e] = -1 - lslot[e];  // equal to T but not taken
      });
  ordered_compact<NT, 4>(
      Lc, wcnt, [&](int e, int&) { return lslot[e] >= 0 && okey(lval[e]) >= T; },
      [&](int r, int e, int) {
        if (r < k) out[r] = rv.key_of(lslot[e]);
      });
}

// Exact selection straight from global memory (heavy ties): 8-bit radix passes
// over the row, then a stable compaction chunk by chunk.  `scratch` holds NBINS ints.
template <int NT, bool KEPT>
__device__ __forceinline__ void fallback_select(const RowView<KEPT> rv, int k, int* scratch, int* wcnt, int* h256,
                                                int* scan_tmp, int* sh, int32_t* out) {
  constexpr int VF = NBINS / (4 * NT) < 4 ? NBINS / (4 * NT) : 4;  // chunk of 4*VF*NT <= NBINS positions
  unsigned pref = 0u, pmask = 0u;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int t = threadIdx.x; t < 256; t += NT) h256[t] = 0;
    __syncthreads();
    for (int base = 0; base < rv.n_slots; base += 16 * NT) {
      int sc[4][4];
      unsigned m[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int s0 = base + 4 * (v * NT + (int)threadIdx.x);
        m[v] = s0 < rv.n_slots ? rv.load4(s0, sc[v]) : 0u;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((m[v] >> c) & 1u) {
            const unsigned u = okey(sc[v][c]);
            if ((u & pmask) == pref) atomicAdd(&h256[(u >> shift) & 255u], 1);
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
    need -= sh[1];
    pref |= (unsigned)sh[0] << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const unsigned T = pref;
  const int need_eq = need;
  int eq_before = 0, written = 0;
  for (int base = 0; base < rv.n_slots; base += 4 * VF * NT) {
    const int hi = min(base + 4 * VF * NT, rv.n_slots);
    int* eq_rank = scratch;  // indexed by position - base
    const int neq = ordered_compact4<NT, VF>(
        base, hi, wcnt, 0,
        [&](int s0, int (&pl)[4]) {
          int sc[4];
          unsigned m = rv.load4(s0, sc), r = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) r |= (((m >> c) & 1u) && okey(sc[c]) == T ? 1u : 0u) << c;
          return r;
        },
        [&](int r, int s, int) { eq_rank[s - base] = r; });
    const int wr = ordered_compact4<NT, VF>(
        base, hi, wcnt, 0,
        [&](int s0, int (&pl)[4]) {
          int sc[4];
          unsigned m = rv.load4(s0, sc), r = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const unsigned u = okey(sc[c]);
            const bool take = ((m >> c) & 1u) && (u > T || (u == T && eq_before + eq_rank[s0 + c - base] < need_eq));
            r |= (take ? 1u : 0u) << c;
          }
          return r;
        },
        [&](int r, int s, int) {
          if (written + r < k) out[written + r] = rv.key_of(s);
        });
    eq_before += neq;
    written += wr;
  }
}

// Rows with no more candidates than k: all of them, in order, then -1 padding.
template <int NT, bool KEPT>
__device__ __forceinline__ void select_all(const RowView<KEPT> rv, int n_valid, int k, int* wcnt, int32_t* out) {
  ordered_compact4<NT, 4>(
      0, rv.n_slots, wcnt, 0,
      [&](int s0, int (&pl)[4]) {
        unsigned m = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) m |= (rv.valid(s0 + c) ? 1u : 0u) << c;
        return m;
      },
      [&](int r, int s, int) {
        if (r < k) out[r] = rv.key_of(s);
      });
  for (int t = n_valid + (int)threadIdx.x; t < k; t += NT) out[t] = -1;
}

// Row setup shared by the kernels: position, slot count, kept table, candidate count.
template <int NT, bool KEPT>
__device__ __forceinline__ RowView<KEPT> make_row(const int32_t* scores, long long ld, const int32_t* q_pos,
                                                  const int32_t* kept, int bs, int n_keep, int L_max, long long row,
                                                  int* kept_s, int* scan_tmp, int* n_valid) {
  RowView<KEPT> rv;
  rv.p = min(q_pos[row], L_max - 1);
  rv.srow = scores + row * ld;
  rv.vec = (((uintptr_t)rv.srow) & 15u) == 0;
  rv.set_block_size(bs);
  if constexpr (KEPT) {
    for (int t = threadIdx.x; t < n_keep; t += NT) kept_s[t] = kept[row * n_keep + t];
    __syncthreads();
    rv.kept_s = kept_s;
    rv.n_slots = (rv.p >= 0) ? n_keep * bs : 0;
    int c = 0;
    if ((int)threadIdx.x < n_keep && rv.p >= 0) {
      const int blk = kept_s[threadIdx.x];
      if (blk >= 0) c = max(0, min(bs, rv.p - blk * bs + 1));
    }
    int tot;
    (void)block_exclusive_scan<NT>(c, scan_tmp, &tot);
    *n_valid = tot;
  } else {
    rv.kept_s = nullptr;
    rv.n_slots = max(rv.p + 1, 0);
    *n_valid = rv.n_slots;
  }
  return rv;
}

// The exact top-k of one row -- the k best candidates by (score desc, slot asc), written
// as keys (rv.key_of) in ascending order, -1 padded -- by one workgroup, from the row's
// scores behind rv (global memory or LDS).  lds_big: NBINS ints; wcnt: 2 * 4 * NT/64.
template <int NT, bool KEPT>
__device__ __forceinline__ void select_row(const RowView<KEPT>& rv, int n_valid, int k, int32_t* out,
                                           int* lds_big, int* wcnt, int* scan_tmp, int* h256, int* sh) {
  constexpr int VG = 4;  // groups of 4 slots per thread per pass
  if (n_valid <= k) {
    select_all<NT, KEPT>(rv, n_valid, k, wcnt, out);
    return;
  }
  for (int t = threadIdx.x; t < NBINS; t += NT) lds_big[t] = 0;
  __syncthreads();
  row_histogram<NT, VG, KEPT>(rv, 0, rv.n_slots, lds_big);
  __syncthreads();
  find_cut_bin<NT>(lds_big, k, scan_tmp, sh);
  const int bstar = sh[4], above = sh[5], cnt_star = sh[6];
  __syncthreads();
  if (above + cnt_star <= CAP) {
    int* lslot = lds_big;
    int* lval = lds_big + CAP;
    const int Lc = ordered_compact4<NT, VG>(
        0, rv.n_slots, wcnt, 0,
        [&](int s0, int (&pl)[4]) {
          unsigned m = rv.load4(s0, pl), r = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) r |= (((m >> c) & 1u) && coarse_bin(pl[c]) >= bstar ? 1u : 0u) << c;
          return r;
        },
        [&](int r, int s, int sc) {
          if (r < CAP) {
            lslot[r] = s;
            lval[r] = sc;
          }
        });
    finish_from_list<NT, KEPT>(rv, Lc, lslot, lval, bstar, above, k, wcnt, h256, scan_tmp, sh, out);
  } else {
    fallback_select<NT, KEPT>(rv, k, lds_big, wcnt, h256, scan_tmp, sh, out);
  }
}

// ---------------------------------------------------------------------------------
// Single workgroup per row (many rows: prefill chunks).
template <int NT, bool KEPT>
__global__ __launch_bounds__(NT) void topk_kernel(const int32_t* __restrict__ scores, long long ld,
                                                  const int32_t* __restrict__ q_pos,
                                                  const int32_t* __restrict__ kept, int bs, int n_keep,
                                                  int L_max, int k, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ count,
                                                  const int32_t* __restrict__ row_state, int n_q, Pages pg) {
  constexpr int NW = NT / 64;
  constexpr int VG = 4;  // groups of 4 slots per thread per pass
  __shared__ int lds_big[NBINS];  // histogram, then the candidate list (slots | scores)
  __shared__ int wcnt[2 * VG * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int kept_s[256];
  __shared__ int sh[8];

  const long long row = blockIdx.x;
  if (row_state != nullptr && row_state[row] == 0) return;  // selected from its candidate list
  int32_t* out = idx + row * (long long)k;
  int n_valid;
  RowView<KEPT> rv = make_row<NT, KEPT>(scores, ld, q_pos, kept, bs, n_keep, L_max, row, kept_s, scan_tmp, &n_valid);
  if constexpr (!KEPT) {
    if (pg.page_table != nullptr) {  // paged caches: the list receives pool rows
      rv.pt = pg.page_table + (row / n_q) * pg.max_pages;
      rv.plog2 = pg.page_log2;
      rv.n_pages = pg.n_pages;
    }
  }
  if (count != nullptr && threadIdx.x == 0) count[row] = min(k, n_valid);
  select_row<NT, KEPT>(rv, n_valid, k, out, lds_big, wcnt, scan_tmp, h256, sh);
}

// ---------------------------------------------------------------------------------
// Two-stage token stage and its top-k in one kernel: one query per workgroup scores the
// slots of its kept blocks (slot s is key kept[s / bs] * bs + s % bs) as the direct
// indexer kernel does -- 64-slot groups straight into MFMA B fragments through a register
// ring, scores into LDS -- and then takes its exact top-k from those LDS scores with the
// score-table kernel's row selection (select_row), so no score table is written or
// read back.  Rows of at most KSEL_SLOTS slots (n_keep * bs).
// GB (bs a multiple of 64): a 64-slot group lies in one kept block, so one wave-uniform
// lookup of that block gives the keys of the whole group (no per-slot division).
// PAGED: k_idx is a pool of pages of 2^page_log2 >= 64 keys behind the sequence's page
// table (a 64-aligned group of keys lies in one page); the list receives pool rows.
// IL (with GB): the keys are read from their chunk-interleaved copy kil (one per
// sequence, kidx_interleave_kernel), whose fragment loads move whole 64-byte pieces per
// quad of lanes (at the token stage's 16 MiB of keys the reads are then bound by the
// Infinity Cache rather than by the texture data path).
template <int D, int MT, bool GB, bool PAGED, bool IL>
__global__ __launch_bounds__(256, 2) void idx_kept_select_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx, const int8_t* __restrict__ kil,
    const int32_t* __restrict__ w, int w_per_query, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ kept, int bs, int n_keep, int n_q, int L_max, int H_I, int k,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, Pages pg) {
  constexpr int NT = 256, NW = NT / 64, KS = D / 64, RING = 4;
  static_assert(!IL || GB, "the interleaved keys are read a 64-key group at a time");
  __shared__ int kept_s[256];
  __shared__ __attribute__((aligned(16))) int sbuf[KSEL_SLOTS];
  __shared__ int lds_big[NBINS];
  __shared__ int wcnt[2 * 4 * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int sh[8];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long row = blockIdx.x;
  const int b = (int)(row / n_q);
  int32_t* out = idx + row * (long long)k;
  v4i A[MT][KS];
  int wv[MT][4];
  issue_query<D, MT>(q_idx, w, w_per_query, row, H_I, A, wv);
  const int p = min(q_pos[row], L_max - 1);
  if (p < 0) {  // no key to see (uniform)
    for (int t = tid; t < k; t += NT) out[t] = -1;
    if (count != nullptr && tid == 0) count[row] = 0;
    return;
  }
  for (int t = tid; t < n_keep; t += NT) kept_s[t] = kept[row * n_keep + t];
  __syncthreads();
  const int n_slots = n_keep * bs;
  int n_valid;  // candidates: keys of kept blocks at or below p
  {
    int c = 0;
    if (tid < n_keep) {
      const int blk = kept_s[tid];
      if (blk >= 0) c = max(0, min(bs, p - blk * bs + 1));
    }
    (void)block_exclusive_scan<NT>(c, scan_tmp, &n_valid);
  }
  const int8_t* kb = k_idx + (PAGED ? 0ll : (long long)b * L_max * D);
  const int8_t* kil_b = IL ? kil + (long long)b * ((L_max + 63) >> 6) * 64 * D : nullptr;
  const int32_t* pt = PAGED ? pg.page_table + (long long)b * pg.max_pages : nullptr;
  const int pmask = PAGED ? (1 << pg.page_log2) - 1 : 0;
  // pool row of logical key j (paged caches; page ids clamped into the pool).  The own
  // block may run past the last page (its keys there are never candidates): the page
  // index is clamped into the sequence's table.
  auto pool_row = [&](int j) -> long long {
    const int pi = min(j >> pg.page_log2, pg.max_pages - 1);
    return ((long long)min(max(pt[pi], 0), pg.n_pages - 1) << pg.page_log2) | (j & pmask);
  };
  // a slot without a kept block, or past the cache, reads a fallback row: its score is
  // never a candidate, and the loads stay unconditional
  auto key_load = [&](int sl) -> long long {
    const int blk = kept_s[sl / bs];
    const int j = blk >= 0 ? min(blk * bs + sl % bs, L_max - 1) : 0;
    if constexpr (PAGED) return pool_row(j);
    return j;
  };
  const int n_groups = (n_slots + 63) / 64;
  const int n_iter = ((n_groups + NW - 1) / NW + RING - 1) / RING * RING;  // groups per wave, padded
  v4i ring[RING][4][KS];
  auto load_group = [&](int i, v4i (&Bf)[4][KS]) {
    const int sg = 64 * (wave + NW * i);
    if constexpr (GB) {
      // groups past the last slot re-read the last group (n_slots is a multiple of 64)
      const int sgc = min(sg, n_slots - 64);
      const int bi = sgc / bs;
      const int blk = kept_s[bi];
      const int base = blk >= 0 ? blk * bs + (sgc - bi * bs) : 0;
      if constexpr (IL) {
        // group base / 64 of the interleaved copy: piece c of key 16 nt + r16 at
        // ((group * D / 16 + c) * 64 + 16 nt + r16) * 16
        const int8_t* kg = kil_b + (long long)(base >> 6) * 64 * D + 16 * r16;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kg + (kchunk<D>(g, ks) * 64 + 16 * nt) * 16);
      } else {
        // paged: the group's 64 keys lie in the page of its first key (base and the page
        // size are multiples of 64)
        const long long rbase = PAGED ? pool_row(base) : (long long)base;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int8_t* kr =
              kb + (PAGED ? rbase + 16 * nt + r16 : (long long)min(base + 16 * nt + r16, L_max - 1)) * D;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kr + 16 * kchunk<D>(g, ks));
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int8_t* kr = kb + key_load(min(sg + 16 * nt + r16, n_slots - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kr + 16 * kchunk<D>(g, ks));
      }
    }
  };
  // the prologue issues the slots in ring order (the loop's waits assume slot 0 is the
  // oldest; a reordered prologue makes the compiler drain every load at the loop head)
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    load_group(r, ring[r]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int wt[MT][4];
  query_weights<MT>(wv, H_I, true, wt);
  for (int i0 = 0; i0 < n_iter; i0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int sg = 64 * (wave + NW * (i0 + r));
      int part[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        v4i acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] = v4i{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma_i8(A[mt][ks], ring[r][nt][ks], acc[mt]);
        }
        int ps = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ps = relu_mad24(acc[mt][e], wt[mt][e], ps);
        part[nt] = ps;
      }
      // the slot just used takes the group RING ahead; the barrier keeps these loads
      // here (left free, the scheduler sinks them towards their MFMAs, and every group
      // then waits for its own loads)
      __builtin_amdgcn_sched_barrier(0);
      load_group(i0 + r + RING, ring[r]);
      __builtin_amdgcn_sched_barrier(0);
      const int res = reduce_scatter4(part);
      const int sl = sg + 16 * g + r16;
      if (sl < n_slots) sbuf[sl] = res;
    }
  }
  __syncthreads();
  RowView<true> rv;
  rv.srow = sbuf;
  rv.kept_s = kept_s;
  rv.n_slots = n_slots;
  rv.p = p;
  rv.set_block_size(bs);
  rv.vec = true;
  if constexpr (PAGED) {  // the list receives pool rows
    rv.pt = pt;
    rv.plog2 = pg.page_log2;
    rv.n_pages = pg.n_pages;
  }
  if (count != nullptr && tid == 0) count[row] = min(k, n_valid);
  select_row<NT, true>(rv, n_valid, k, out, lds_big, wcnt, scan_tmp, h256, sh);
}

// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int MT>
static hipError_t launch_kept_select_t(const IdxArgs& a, int k, int32_t* idx, int32_t* count, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  const bool gb = a.block_size % 64 == 0, paged = a.pages.page_table != nullptr, il = gb && a.k_il != nullptr;
#define LSA_KSEL(GB, PG, IL)                                                                                        \
  hipLaunchKernelGGL((idx_kept_select_kernel<D, MT, GB, PG, IL>), dim3((unsigned)rows), dim3(256), 0, st, a.q_idx, \
                     a.k_idx, a.k_il, a.w, a.w_per_query, a.q_pos, a.kept, a.block_size, a.n_keep, a.n_q, a.L_max, \
                     a.H_I, k, idx, count, a.pages)
  if (il && paged) LSA_KSEL(true, true, true);
  else if (il) LSA_KSEL(true, false, true);
  else if (gb && paged) LSA_KSEL(true, true, false);
  else if (gb) LSA_KSEL(true, false, false);
  else if (paged) LSA_KSEL(false, true, false);
  else LSA_KSEL(false, false, false);
#undef LSA_KSEL
  return hipGetLastError();
}

// Chunk-interleaved index keys for the token stage.  An MFMA fragment of 16 keys takes
// 16 bytes of each key per lane, lanes 0..15 on 16 different keys; loaded from key rows,
// every quad of lanes touches four rows, and such loads deliver about a quarter of the
// bytes per cycle that loads of contiguous lanes do.  Here group G of 64 keys of a
// sequence stores, for each 16-byte piece c of the key rows, the 64 keys' pieces side by
// side -- il[b][G][c][jj] = k_idx[b][64 G + jj][16 c .. 16 c + 15] -- so the 16 keys of a
// fragment are 256 contiguous bytes per piece.  Keys at or past L_max are zero.  One
// thread per 16-byte piece, in output order (coalesced writes).
template <int D>
__global__ __launch_bounds__(256) void kidx_interleave_kernel(const int8_t* __restrict__ k_idx, int L_max,
                                                              long long n_grp, long long total, Pages pg,
                                                              v4i* __restrict__ out) {
  constexpr int CH = D / 16;
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < total; t += (long long)gridDim.x * 256) {
    const int jj = (int)(t & 63);
    const long long q = t >> 6;
    const int c = (int)(q % CH);
    const long long gq = q / CH;
    const long long b = gq / n_grp;
    const long long j = (gq - b * n_grp) * 64 + jj;
    v4i v = v4i{0, 0, 0, 0};
    if (j < L_max) {
      long long r;
      if (pg.page_table != nullptr) {  // page ids clamped into the pool
        const int pi = (int)(j >> pg.page_log2);
        const int page = min(max(pg.page_table[b * pg.max_pages + pi], 0), pg.n_pages - 1);
        r = ((long long)page << pg.page_log2) | (j & ((1 << pg.page_log2) - 1));
      } else {
        r = b * L_max + j;
      }
      v = *(const v4i*)(k_idx + r * D + 16 * c);
    }
    out[t] = v;
  }
}

// ---------------------------------------------------------------------------------
// Several workgroups per row (few long rows: decode); workspace layout: SegWs.

// clears the histogram, the group sums and the arrival counter of every row
__global__ void topk_seg_zero_kernel(int* ws, long long row_ints, long long rows) {
  const long long r = blockIdx.y;
  if (r >= rows) return;
  int* h = ws + r * row_ints;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < NBINS + INFO + NGRP; t += gridDim.x * blockDim.x)
    h[t] = 0;
}

template <int NT, bool KEPT>
__global__ __launch_bounds__(NT) void topk_seg_hist_kernel(const int32_t* __restrict__ scores, long long ld,
                                                           const int32_t* __restrict__ q_pos,
                                                           const int32_t* __restrict__ kept, int bs, int n_keep,
                                                           int L_max, int k, SegWs ws) {
  constexpr int NW = NT / 64;
  __shared__ int hist[NBINS];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int kept_s[256];
  const long long row = blockIdx.y;
  const int seg = blockIdx.x;
  int n_valid;
  const RowView<KEPT> rv = make_row<NT, KEPT>(scores, ld, q_pos, kept, bs, n_keep, L_max, row, kept_s, scan_tmp, &n_valid);
  const int lo = seg * SEG, hi = min(lo + SEG, rv.n_slots);
  if (n_valid <= k) return;
  const int n_seg_row = (rv.n_slots + SEG - 1) / SEG;
  if (lo >= hi) return;  // segments past the row's end do not take part
  for (int t = threadIdx.x; t < NBINS; t += NT) hist[t] = 0;
  __syncthreads();
  row_histogram<NT, 8, KEPT>(rv, lo, hi, hist);
  __syncthreads();
  __shared__ int sh[8];
  merge_row_histogram<NT>(hist, ws.hist(row), ws.info(row), n_seg_row, k, scan_tmp, sh);
}

// One segment of a flat row: the entries of bins >= b* go, in slot order, to the
// segment's candidate list in the workspace.  Every load the workgroup needs is
// issued before any of them is used -- the row's position, its cut and the
// segment's scores (read up to L_max and masked by the position afterwards).
template <int NT>
__global__ __launch_bounds__(NT) void topk_seg_select_kernel(const int32_t* __restrict__ scores, long long ld,
                                                             const int32_t* __restrict__ q_pos, int L_max, int k,
                                                             SegWs ws) {
  constexpr int NW = NT / 64;
  constexpr int V = SEG / (4 * NT);  // one pass covers the segment
  static_assert(4 * V * NT == SEG, "segment = one compaction pass");
  __shared__ int wcnt[V * NW];
  const long long row = blockIdx.y;
  const int seg = blockIdx.x;
  const int lo = seg * SEG, hi_max = min(lo + SEG, L_max);
  const int32_t* srow = scores + row * ld;
  const int* info = ws.info(row);

  const int p_raw = q_pos[row];
  const int bstar = info[0], overflow = info[3];
  const bool vec = (((uintptr_t)srow) & 15u) == 0;
  int sc[V][4];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int pos4 = lo + 4 * (v * NT + (int)threadIdx.x);
    if (vec && pos4 + 3 < hi_max) {
      const v4i x = *(const v4i*)(srow + pos4);
      sc[v][0] = x[0]; sc[v][1] = x[1]; sc[v][2] = x[2]; sc[v][3] = x[3];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) sc[v][c] = pos4 + c < hi_max ? srow[pos4 + c] : 0;
    }
  }

  const int n_slots = max(min(p_raw, L_max - 1) + 1, 0);
  if (n_slots <= k) return;  // every candidate is taken: the finish kernel lists them
  const int hi = min(hi_max, n_slots);
  if (lo >= hi) return;
  if (overflow) return;  // the finish kernel selects from global memory
  unsigned m[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int pos4 = lo + 4 * (v * NT + (int)threadIdx.x);
    m[v] = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) m[v] |= (pos4 + c < hi && coarse_bin(sc[v][c]) >= bstar ? 1u : 0u) << c;
  }
  int* cand = ws.cand(row, seg);
  const int n = ordered_emit4<NT, V>(lo, m, sc, wcnt, 0, [&](int r, int s, int v) {
    if (r < CAP) {
      cand[2 * r] = s;
      cand[2 * r + 1] = v;
    }
  });
  if (threadIdx.x == 0) ws.cnt(row)[seg] = n;
}

template <int NT, bool KEPT>
__global__ __launch_bounds__(NT) void topk_seg_finish_kernel(const int32_t* __restrict__ scores, long long ld,
                                                             const int32_t* __restrict__ q_pos,
                                                             const int32_t* __restrict__ kept, int bs, int n_keep,
                                                             int L_max, int k, SegWs ws, int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ count) {
  constexpr int NW = NT / 64;
  __shared__ int lds_big[NBINS];
  __shared__ int wcnt[2 * 4 * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int kept_s[256];
  __shared__ int sh[8];
  __shared__ int seg_off[1025];
  const long long row = blockIdx.x;
  int32_t* out = idx + row * (long long)k;
  // loads that do not depend on each other go out together: the row's cut and its
  // first NT segment counts (read for every segment of the workspace; only the
  // row's own are used), then the row's position
  const int* info = ws.info(row);
  const int bstar = info[0], above = info[1], overflow = info[3];
  const int cnt0 = (int)threadIdx.x < ws.n_seg ? ws.cnt(row)[threadIdx.x] : 0;
  int n_valid;
  const RowView<KEPT> rv = make_row<NT, KEPT>(scores, ld, q_pos, kept, bs, n_keep, L_max, row, kept_s, scan_tmp, &n_valid);
  if (count != nullptr && threadIdx.x == 0) count[row] = min(k, n_valid);
  if (n_valid <= k) {
    select_all<NT, KEPT>(rv, n_valid, k, wcnt, out);
    return;
  }
  if (overflow) {
    fallback_select<NT, KEPT>(rv, k, lds_big, wcnt, h256, scan_tmp, sh, out);
    return;
  }
  // segment offsets (n_seg <= 1024, scanned NT at a time), then the candidates in slot order
  const int n_seg = (rv.n_slots + SEG - 1) / SEG;
  {
    int carry = 0;
    for (int s0 = 0; s0 < n_seg; s0 += NT) {
      const int s = s0 + (int)threadIdx.x;
      const int c = s < n_seg ? (s0 == 0 ? cnt0 : ws.cnt(row)[s]) : 0;
      int tot;
      const int ex = block_exclusive_scan<NT>(c, scan_tmp, &tot);
      if (s < n_seg) seg_off[s] = carry + ex;
      carry += tot;
    }
    if (threadIdx.x == 0) seg_off[n_seg] = carry;
    __syncthreads();
  }
  const int Lc = min(seg_off[n_seg], CAP);
  int* lslot = lds_big;
  int* lval = lds_big + CAP;
  // all candidates of the row in one flat pass, each entry's segment found by binary
  // search in seg_off, G entries per thread in flight (a loop over segments would
  // wait out one memory latency per segment)
  constexpr int G = 8;
  for (int e0 = 0; e0 < Lc; e0 += G * NT) {
    int gs[G], gv[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int ec = min(e0 + u * NT + (int)threadIdx.x, Lc - 1);  // clamped: loads stay unconditional
      int lo = 0, hi = n_seg;  // seg_off[lo] <= ec < seg_off[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seg_off[mid] <= ec) lo = mid;
        else hi = mid;
      }
      const int* cand = ws.cand(row, lo) + 2 * (ec - seg_off[lo]);
      gs[u] = cand[0];
      gv[u] = cand[1];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int e = e0 + u * NT + (int)threadIdx.x;
      if (e < Lc) {
        lslot[e] = gs[u];
        lval[e] = gv[u];
      }
    }
  }
  __syncthreads();
  finish_from_list<NT, KEPT>(rv, Lc, lslot, lval, bstar, above, k, wcnt, h256, scan_tmp, sh, out);
}

// Flat rows whose selection state the decode indexer built (one record per span of
// dec_span(n_valid, parts) keys: band, group sums, band bins, candidate list; no score
// table): one workgroup per row.  The row's group sums are the sum of its spans'; the
// cut group's bins likewise, and b* is the bin holding the k-th best entry.  Every
// entry of bin >= b* is then in its span's list (lbw <= b*: no span holds k entries
// above the cut) or, for a span whose list overflowed (lbw = -1), in its slice of the
// score table; they are gathered in slot order from both.  If they overflow the LDS
// list (heavy ties at b*), the row's table is completed instead -- a list span's
// slice is set to INT_MIN, below every candidate, and its list entries are written
// over it -- and the exact radix fallback runs over the table.
template <int NT>
__global__ __launch_bounds__(NT) void topk_list_finish_kernel(int32_t* __restrict__ scores, long long ld,
                                                              const int32_t* __restrict__ q_pos, int L_max, int k,
                                                              DecWs ws, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ count, int n_q, Pages pg) {
  constexpr int NW = NT / 64;
  constexpr int V = 3;
  static_assert(NT % NGRP == 0 && NT % GRP == 0, "whole groups of threads per group sum and per bin");
  static_assert(NT >= DEC_MAX_PARTS, "one span per thread");
  __shared__ int lds_big[NBINS];
  __shared__ int wcnt[2 * 4 * NW];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int sh[8];
  __shared__ int loff[NT + 1];
  __shared__ int slen[NT];   // per span: entries to gather
  __shared__ int slist[NT];  // per span: 1 = list, 0 = table slice
  __shared__ int sband[2][NT];
  __shared__ const int* ssc[NT];  // per span: its scores (list or table slice)
  __shared__ const int* ssl[NT];  // per span: its list's slots
  __shared__ int sslot0[NT];      // per span: -1 (list) or its first slot (table slice)
  constexpr int TMAX = 1024;      // entries of b* ranked directly
  __shared__ int tb_score[TMAX], tb_slot[TMAX], tb_n;
  __shared__ int gs_l[NGRP];
  __shared__ int bins_l[GRP];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  int32_t* out = idx + row * (long long)k;

  // The position, a span header per thread and the first group sums of every thread
  // are requested together, before the position is known: records of spans past the
  // row's last one (stale) are read but not used.  Thread t adds group t % NGRP of
  // spans t / NGRP, t / NGRP + NT / NGRP, ...
  const int p_raw = q_pos[row];
  const int4 hdr = *reinterpret_cast<const int4*>(ws.hdr(row, min(tid, ws.parts - 1)));
  const int gs0 = ws.gsum(row, min(tid / NGRP, ws.parts - 1))[tid % NGRP];

  RowView<false> rv;
  rv.p = min(p_raw, L_max - 1);
  rv.srow = scores + row * ld;
  rv.vec = (((uintptr_t)rv.srow) & 15u) == 0;
  rv.bs = 0;
  rv.kept_s = nullptr;
  rv.n_slots = max(rv.p + 1, 0);
  if (pg.page_table != nullptr) {
    rv.pt = pg.page_table + (row / n_q) * pg.max_pages;
    rv.plog2 = pg.page_log2;
    rv.n_pages = pg.n_pages;
  }
  const int n_valid = rv.n_slots;
  if (count != nullptr && tid == 0) count[row] = min(k, n_valid);
  if (n_valid <= k) {
    select_all<NT, false>(rv, n_valid, k, wcnt, out);
    return;
  }
  const int span = dec_span(n_valid, ws.parts);
  const int n_sp = (n_valid + span - 1) / span;  // spans of this row (each left a record)
  if (tid < n_sp) {
    sband[0][tid] = hdr.x;
    sband[1][tid] = hdr.y;
    slist[tid] = hdr.w >= 0;
    slen[tid] = hdr.w >= 0 ? hdr.z : min(n_valid, (tid + 1) * span) - tid * span;
  }
  if (tid < NGRP) gs_l[tid] = 0;
  if (tid < GRP) bins_l[tid] = 0;
  {
    int acc = tid / NGRP < n_sp ? gs0 : 0;
    for (int sp = tid / NGRP + NT / NGRP; sp < n_sp; sp += NT / NGRP) acc += ws.gsum(row, sp)[tid % NGRP];
    __syncthreads();
    if (acc) atomicAdd(&gs_l[tid % NGRP], acc);
  }
  __syncthreads();

  // cut: group holding the k-th best entry, then the bin inside it
  {
    const int gs = tid < NGRP ? gs_l[NGRP - 1 - tid] : 0;  // highest group first
    int tot;
    const int excl = block_exclusive_scan<NT>(gs, scan_tmp, &tot);
    if (excl < k && excl + gs >= k) {
      sh[0] = NGRP - 1 - tid;
      sh[1] = excl;
    }
    __syncthreads();
    const int g = sh[0];
    // bin g*GRP + tid % GRP of spans tid / GRP, tid / GRP + NT / GRP, ... (inside their bands)
    const int bin = g * GRP + tid % GRP;
    int acc = 0;
    for (int sp = tid / GRP; sp < n_sp; sp += NT / GRP)
      if (bin >= sband[0][sp] && bin <= sband[1][sp]) acc += ws.hist(row, sp)[bin];
    if (acc) atomicAdd(&bins_l[tid % GRP], acc);
    __syncthreads();
    if (tid < 64) {
      const int hb = lane < GRP ? bins_l[GRP - 1 - lane] : 0;  // highest bin first
      int incl = hb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const unsigned long long hit = __ballot(sh[1] + incl >= k);
      const int first = (int)__ffsll((long long)hit) - 1;
      if (lane == first) {
        sh[4] = g * GRP + GRP - 1 - lane;
        sh[5] = sh[1] + incl - hb;
        sh[6] = hb;
      }
    }
    __syncthreads();
  }
  const int bstar = sh[4], above = sh[5], cnt_star = sh[6];

  if (above + cnt_star > CAP) {
    int32_t* srow = scores + row * ld;
    for (int sp = 0; sp < n_sp; ++sp) {
      if (!slist[sp]) continue;  // uniform: LDS after a barrier
      const int j1 = min(n_valid, (sp + 1) * span);
      for (int j = sp * span + tid; j < j1; j += NT) srow[j] = INT_MIN;
    }
    __syncthreads();
    for (int sp = 0; sp < n_sp; ++sp) {
      if (!slist[sp]) continue;
      const int* Ls = ws.lslot(row, sp);
      const int* Lv = ws.lscore(row, sp);
      for (int e = tid; e < slen[sp]; e += NT) srow[Ls[e]] = Lv[e];
    }
    __syncthreads();
    fallback_select<NT, false>(rv, k, lds_big, wcnt, h256, scan_tmp, sh, out);
    return;
  }

  // Offsets of the spans' sources in their concatenation, each count rounded up to a
  // multiple of 4 (so a thread's quad of consecutive entries lies in one span), and
  // where the entries come from: a list's slot and score arrays, or a table slice of
  // scores (slot = first slot + position).  Then an ordered compaction over the
  // concatenation, a quad per thread and step: two 16-byte loads, all issued before
  // any is used.  The padding entries, and the reads they make, stay inside the list
  // (lcap is a multiple of 4) or the table row (a slice starts at a multiple of 64
  // and the row is a multiple of 64 long).
  int* lslot = lds_big;
  int* lval = lds_big + CAP;
  int n_all;
  {
    const int ex = block_exclusive_scan<NT>(tid < n_sp ? (slen[tid] + 3) & ~3 : 0, scan_tmp, &n_all);
    if (tid < n_sp) {
      loff[tid] = ex;
      ssc[tid] = slist[tid] ? ws.lscore(row, tid) : rv.srow + tid * span;
      ssl[tid] = slist[tid] ? ws.lslot(row, tid) : rv.srow + tid * span;  // slices: read, not used
      sslot0[tid] = slist[tid] ? -1 : tid * span;
    }
    if (tid == 0) tb_n = 0;
    __syncthreads();
  }
  struct SP {
    int slot, score;
  };
  // Each step gives a thread one quad of consecutive entries (4*V*NT entries a step):
  // the span found by a binary search over the offsets, then two 16-byte loads
  // (scores, and a list's slots), all issued before any is used.
  constexpr int STEP = 4 * V * NT;
  struct Quad {
    v4i sc, sl;
    int e0, j0, lim, s0;
  };
  auto load_step = [&](int base, Quad (&q)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      q[v].e0 = base + 4 * (v * NT + tid);
      const int ec = min(q[v].e0, n_all - 4);  // clamped: the loads stay unconditional
      int lo = 0, hi = n_sp;                    // last span with loff[lo] <= ec
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (loff[mid] <= ec) lo = mid;
        else hi = mid;
      }
      q[v].j0 = ec - loff[lo];
      q[v].lim = slen[lo];
      q[v].s0 = sslot0[lo];
      q[v].sc = *reinterpret_cast<const v4i*>(ssc[lo] + q[v].j0);
      q[v].sl = *reinterpret_cast<const v4i*>(ssl[lo] + q[v].j0);
    }
  };
  auto valid = [&](const Quad& q, int c) { return q.e0 < n_all && q.j0 + c < q.lim; };
  auto slot_of = [&](const Quad& q, int c) { return q.s0 < 0 ? q.sl[c] : q.s0 + q.j0 + c; };

  // Pass 1: collect the entries of b* (any order; one LDS atomic per wave and quad
  // slot).  The first step's quads stay in registers for pass 2.
  Quad q0[V];
  load_step(0, q0);
  auto collect = [&](const Quad (&q)[V]) {
    unsigned in = 0;  // bit 4v+c: entry (v, c) is in b*
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) in |= (valid(q[v], c) && coarse_bin(q[v].sc[c]) == bstar ? 1u : 0u) << (4 * v + c);
    // the wave's entries get consecutive places: a prefix sum over the lanes, one atomic
    const int cnt = __popc(in);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int wb = 0;
    if (lane == 63 && incl > 0) wb = atomicAdd(&tb_n, incl);
    int i = __shfl(wb, 63) + incl - cnt;
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((in >> (4 * v + c)) & 1u) {
          if (i < TMAX) {
            tb_score[i] = q[v].sc[c];
            tb_slot[i] = slot_of(q[v], c);
          }
          ++i;
        }
  };
  collect(q0);
  for (int base = STEP; base < n_all; base += STEP) {
    Quad q[V];
    load_step(base, q);
    collect(q);
  }
  __syncthreads();
  const int n_star = tb_n;
  int running = 0, parity = 0;
  if (n_star > TMAX) {
    // Heavy ties at b*: every entry of bin >= b* into the LDS list (fewer than CAP),
    // then the exact selection over it.
    const int thr = bin_floor(bstar);  // coarse_bin(v) >= b*  <=>  v >= thr
    for (int base = 0; base < n_all; base += STEP) {
      Quad q[V];
      load_step(base, q);
      unsigned m[V];
      SP pl[V][4];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        m[v] = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pl[v][c].slot = slot_of(q[v], c);
          pl[v][c].score = q[v].sc[c];
          m[v] |= (valid(q[v], c) && q[v].sc[c] >= thr ? 1u : 0u) << c;
        }
      }
      running = ordered_emit4<NT, V>(base, m, pl, wcnt + parity * V * NW, running, [&](int r, int, SP x) {
        if (r < CAP) {
          lslot[r] = x.slot;
          lval[r] = x.score;
        }
      });
      parity ^= 1;
    }
    __syncthreads();
    finish_from_list<NT, false>(rv, min(running, CAP), lslot, lval, bstar, above, k, wcnt, h256, scan_tmp, sh,
                                out);
    return;
  }

  // The cutoff: the (k - above)-th best entry of b* by (score desc, slot asc), found by
  // one wave among the collected ones.
  if (tid < 64) {
    unsigned long long kpref;
    const unsigned long long kmask = bin_key_prefix(bstar, &kpref);
    const auto key = [&](int i) {
      return ((unsigned long long)okey(tb_score[i]) << 32) | (0xFFFFFFFFu - (unsigned)tb_slot[i]);
    };
    const unsigned long long cut =
        n_star <= 256 ? wave_select_kth<4>(n_star, k - above, key, h256, kpref, kmask)
                      : wave_select_kth<TMAX / 64>(n_star, k - above, key, h256, kpref, kmask);
    if (tid == 0) {
      sh[0] = (int)((unsigned)(cut >> 32) ^ 0x80000000u);
      sh[1] = (int)(0xFFFFFFFFu - (unsigned)cut);
    }
  }
  __syncthreads();
  const int T = sh[0], slot_T = sh[1];

  // Pass 2: the taken entries -- score > T, or score == T and slot <= slot_T; exactly
  // k of them -- straight to the output in slot order.
  auto emit = [&](int base, const Quad (&q)[V]) {
    unsigned m[V];
    SP pl[V][4];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v] = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int sc = q[v].sc[c], sl = slot_of(q[v], c);
        pl[v][c].slot = sl;
        pl[v][c].score = sc;
        m[v] |= (valid(q[v], c) && (sc > T || (sc == T && sl <= slot_T)) ? 1u : 0u) << c;
      }
    }
    running = ordered_emit4<NT, V>(base, m, pl, wcnt + parity * V * NW, running, [&](int r, int, SP x) {
      if (r < k) out[r] = rv.key_of(x.slot);
    });
    parity ^= 1;
  };
  emit(0, q0);
  for (int base = STEP; base < n_all; base += STEP) {
    Quad q[V];
    load_step(base, q);
    emit(base, q);
  }
}

// Threshold of each flat row for the thresholded selection (one workgroup per row).
// A row of at most t.row_min keys keeps the score table (state 1).  Otherwise its
// threshold is the t-th best of its m sampled scores (keys 0, stride, 2*stride, ... up
// to the query position), t = ceil(2k * m / n_valid) (at most m), so about 2k entries
// of the row are expected to reach it; the selection stays exact whatever the sample
// shows (rows that fall short of k or overflow take the table path).
template <int NT>
__global__ __launch_bounds__(NT) void thr_kernel(const int32_t* __restrict__ samp, long long ld_s,
                                                 const int32_t* __restrict__ q_pos, int L_max, int k, int stride,
                                                 int mode, ThrArgs t) {
  constexpr int NW = NT / 64;
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int sh[8];
  const long long row = blockIdx.x;
  const int p = min(q_pos[row], L_max - 1);
  const int n_valid = max(p + 1, 0);
  int32_t* theta = const_cast<int32_t*>(t.theta);
  if (n_valid <= t.row_min) {
    if (threadIdx.x == 0) {
      theta[row] = INT_MIN;
      t.rstate[row] = 1;
      t.cnt[row] = 0;
    }
    return;
  }
  int th;
  if (mode == 1) {
    th = INT_MAX;
  } else if (mode == 2) {
    th = INT_MIN;
  } else {
    const int m = p / stride + 1;
    const long long tt = (2LL * k * m + n_valid - 1) / n_valid;
    const int need = (int)min<long long>(m, max<long long>(1, tt));
    const int32_t* srow = samp + row * ld_s;
    int need_eq;
    const unsigned T = radix_select32<NT, 4>(
        m, need, h256, scan_tmp, sh,
        [&](int pos, int& sc) {
          sc = srow[pos];
          return true;
        },
        &need_eq);
    th = (int)(T ^ 0x80000000u);
  }
  if (threadIdx.x == 0) {
    theta[row] = th;
    t.rstate[row] = 0;
    t.cnt[row] = 0;
  }
}

// The need-th largest of the 64-bit keys kv[j][c] with bit 4j+c of take[j / 8] set
// (1 <= need <= their count), exactly, by the whole workgroup: 8-bit radix passes
// from the highest bit not fixed by pmask0 (every taken key agrees with pref0 there).
template <int NT, int J>
__device__ __forceinline__ unsigned long long block_select_kth64(const unsigned long long (&kv)[J][4],
                                                                 const unsigned (&take)[(J + 7) / 8], int need,
                                                                 int* h256, int* scan_tmp, int* sh,
                                                                 unsigned long long pref0,
                                                                 unsigned long long pmask0) {
  static_assert(NT >= 256, "one bucket per thread in the scan");
  const int hb = pmask0 == ~0ull ? -1 : 63 - __clzll((long long)~pmask0);
  if (hb < 0) return pref0;
  int shift = (hb / 8) * 8;
  unsigned long long pmask = shift + 8 >= 64 ? 0ull : ~((1ull << (shift + 8)) - 1ull);
  unsigned long long pref = pref0 & pmask;
  const int t = threadIdx.x;
  for (; shift >= 0; shift -= 8) {
    if (t < 256) h256[t] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (((take[j / 8] >> (4 * (j % 8) + c)) & 1u) && (kv[j][c] & pmask) == pref)
          atomicAdd(&h256[(int)((kv[j][c] >> shift) & 255ull)], 1);
    __syncthreads();
    const int cnt = t < 256 ? h256[255 - t] : 0;
    int tot;
    const int excl = block_exclusive_scan<NT>(cnt, scan_tmp, &tot);
    if (t < 256 && excl < need && excl + cnt >= need) {
      sh[0] = 255 - t;
      sh[1] = excl;
    }
    __syncthreads();
    need -= sh[1];
    pref |= (unsigned long long)sh[0] << shift;
    pmask |= 255ull << shift;
    __syncthreads();
  }
  return pref;
}

// Exact top-k of a list row from its candidate list (one workgroup per row): every
// entry of the row with score >= its threshold is in the list, and there are at
// least k of them, so the row's top-k by (score desc, slot asc) is the list's.
// The list stays in registers (thread t holds quads t, t + NT, ...).  One pass builds
// the coarse-bin histogram and finds the bin b* of the k-th best; the entries of b*
// are gathered in LDS and one wave finds the cutoff among them (the whole workgroup
// when b* holds more than TMAX, i.e. heavy ties); the taken entries are marked in a
// bitmap of the row's slots (sharing the histogram's LDS) and written in ascending
// order.  A list that fell short of k or overflowed marks its row for the score table.
// Dynamic LDS: max(NBINS, ceil(L_max / 32)) ints.
template <int NT, int J>
__global__ __launch_bounds__(NT) void list_topk_kernel(const int32_t* __restrict__ q_pos, int L_max, int k,
                                                       ThrArgs t, int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count, int n_q, Pages pg) {
  constexpr int NW = NT / 64;
  constexpr int TMAX = 512;
  constexpr int JW = (J + 7) / 8;
  extern __shared__ int lds_dyn[];
  __shared__ int tb_score[TMAX], tb_slot[TMAX];
  __shared__ int scan_tmp[NW + 1];
  __shared__ int h256[256];
  __shared__ int sh[8];
  __shared__ int tb_n;
  int* hist = lds_dyn;
  unsigned* bm = reinterpret_cast<unsigned*>(lds_dyn);
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  if (t.rstate[row] != 0) return;
  const int n_valid = max(min(q_pos[row], L_max - 1) + 1, 0);
  const int c = t.cnt[row];
  if (c < k || c > t.cap) {
    if (tid == 0) t.rstate[row] = 2;
    return;
  }
  int32_t* out = idx + row * (long long)k;
  if (count != nullptr && tid == 0) count[row] = k;  // a list row has more than cap >= k keys
  // the list: cap is a multiple of 4, so each row's arrays are 16-byte aligned
  const int32_t* lsl = t.lslot + row * t.cap;
  const int32_t* lsc = t.lscore + row * t.cap;
  v4i sc[J], sl[J];
  unsigned valid[JW];
#pragma unroll
  for (int w = 0; w < JW; ++w) valid[w] = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e0 = 4 * (tid + NT * j);
    if (e0 < c) {
      sc[j] = *reinterpret_cast<const v4i*>(lsc + e0);
      sl[j] = *reinterpret_cast<const v4i*>(lsl + e0);
#pragma unroll
      for (int q = 0; q < 4; ++q) valid[j / 8] |= (e0 + q < c ? 1u : 0u) << (4 * (j % 8) + q);
    } else {
      sc[j] = v4i{0, 0, 0, 0};
      sl[j] = v4i{0, 0, 0, 0};
    }
  }
  auto is_valid = [&](int j, int q) { return ((valid[j / 8] >> (4 * (j % 8) + q)) & 1u) != 0u; };
  for (int b = tid; b < NBINS; b += NT) hist[b] = 0;
  if (tid == 0) tb_n = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (is_valid(j, q)) atomicAdd(&hist[coarse_bin(sc[j][q])], 1);
  __syncthreads();
  find_cut_bin<NT>(hist, k, scan_tmp, sh);
  const int bstar = sh[4], above = sh[5], n_star = sh[6];
  const int need = k - above;  // 1 <= need <= n_star
  unsigned long long kpref;
  const unsigned long long kmask = bin_key_prefix(bstar, &kpref);
  auto key_of = [](int score, int slot) {
    return ((unsigned long long)okey(score) << 32) | (0xFFFFFFFFu - (unsigned)slot);
  };
  unsigned long long cut;
  if (n_star <= TMAX) {
    // gather b* (any order): a prefix sum over the wave's lanes, one LDS atomic a wave
    unsigned in[JW];
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < JW; ++w) in[w] = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (is_valid(j, q) && coarse_bin(sc[j][q]) == bstar) {
          in[j / 8] |= 1u << (4 * (j % 8) + q);
          ++cnt;
        }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int wb = 0;
    if (lane == 63 && incl > 0) wb = atomicAdd(&tb_n, incl);
    int i = __shfl(wb, 63) + incl - cnt;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((in[j / 8] >> (4 * (j % 8) + q)) & 1u) {
          tb_score[i] = sc[j][q];
          tb_slot[i] = sl[j][q];
          ++i;
        }
    __syncthreads();
    if (tid < 64) {
      const auto key = [&](int e) { return key_of(tb_score[e], tb_slot[e]); };
      const unsigned long long r = n_star <= 256 ? wave_select_kth<4>(n_star, need, key, h256, kpref, kmask)
                                                 : wave_select_kth<TMAX / 64>(n_star, need, key, h256, kpref, kmask);
      if (tid == 0) {
        sh[0] = (int)(unsigned)(r >> 32);
        sh[1] = (int)(unsigned)r;
      }
    }
    __syncthreads();
    cut = ((unsigned long long)(unsigned)sh[0] << 32) | (unsigned)sh[1];
  } else {
    // heavy ties: the keys of b* stay in registers for a workgroup-wide radix select
    unsigned long long kv[J][4];
    unsigned in[JW];
#pragma unroll
    for (int w = 0; w < JW; ++w) in[w] = 0u;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kv[j][q] = key_of(sc[j][q], sl[j][q]);
        if (is_valid(j, q) && coarse_bin(sc[j][q]) == bstar) in[j / 8] |= 1u << (4 * (j % 8) + q);
      }
    cut = block_select_kth64<NT, J>(kv, in, need, h256, scan_tmp, sh, kpref, kmask);
  }
  // the taken entries (key >= cut; exactly k of them) into the bitmap of slots
  const int nw = (n_valid + 31) / 32;
  for (int wd = tid; wd < nw; wd += NT) bm[wd] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (is_valid(j, q) && key_of(sc[j][q], sl[j][q]) >= cut) {
        const int s = sl[j][q];
        atomicOr(&bm[s >> 5], 1u << (s & 31));
      }
  __syncthreads();
  // ascending output: thread tid takes words [tid * WPT, tid * WPT + WPT)
  const int WPT = (nw + NT - 1) / NT;
  int my = 0;
  for (int i = 0; i < WPT; ++i) {
    const int wd = tid * WPT + i;
    if (wd < nw) my += __popc(bm[wd]);
  }
  int tot;
  int r = block_exclusive_scan<NT>(my, scan_tmp, &tot);
  for (int i = 0; i < WPT; ++i) {
    const int wd = tid * WPT + i;
    if (wd >= nw) break;
    unsigned m = bm[wd];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (r < k) {
        const int key = wd * 32 + bit;
        // paged caches: the key's pool row
        out[r] = pg.page_table == nullptr
                     ? key
                     : (min(max(pg.page_table[(row / n_q) * pg.max_pages + (key >> pg.page_log2)], 0), pg.n_pages - 1)
                        << pg.page_log2) | (key & ((1 << pg.page_log2) - 1));
      }
      ++r;
    }
  }
}

// The best n_sel of a row's n_sc > n_sel scored blocks by (int64 score desc, block asc),
// written ascending to out[0..n_sel): one pass for the keys' max and min, one per 8-bit
// radix digit below the prefix they share, one to rank the blocks equal to the cut and
// one to write; every pass re-reads the row.  Returns n_sel.  All threads call.
template <int NT>
__device__ int blk_cut_passes(const long long* __restrict__ br, int n_sc, int n_sel, int32_t* __restrict__ out) {
  constexpr int V = 4;
  __shared__ int wcnt[2 * V * (NT / 64)];
  __shared__ int scan_tmp[NT / 64 + 1];
  __shared__ int h256[256];
  __shared__ unsigned long long shu[4];
  __shared__ int sh[4];
  __shared__ int drop_from;
  const int tid = threadIdx.x;
  auto key64 = [&](int m) -> unsigned long long {
    return (unsigned long long)br[m] ^ 0x8000000000000000ull;
  };
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
  if (tid == 0) drop_from = n_sc;
  __syncthreads();
  ordered_compact<NT, V>(n_sc, wcnt, [&](int m, int&) { return key64(m) == T; },
                         [&](int r, int m, int) {
                           if (r == need_eq) drop_from = m;
                         });
  const int df = drop_from;
  return ordered_compact<NT, V>(
      n_sc, wcnt,
      [&](int m, int&) {
        const unsigned long long u = key64(m);
        return u > T || (u == T && m < df);
      },
      [&](int r, int m, int) {
        if (r < n_sel) out[r] = m;
      });
}

// Block keep of the two-stage indexer: own block + the best n_keep-1 earlier blocks
// by (int64 score desc, block asc), ascending, -1 padded.
template <int NT>
__global__ __launch_bounds__(NT) void blk_select_kernel(const long long* __restrict__ bscores, long long ld,
                                                        const int32_t* __restrict__ q_pos, int n_blocks,
                                                        int bs, int n_keep, int32_t* __restrict__ kept,
    const int32_t* __restrict__ rstate) {
  constexpr int V = 4;
  __shared__ int wcnt[2 * V * (NT / 64)];
  const long long row = blockIdx.x;
  if (rstate != nullptr && rstate[row] == 0) return;  // kept from its list
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
  const int n_sel = min(n_keep - 1, n_sc);
  int written = 0;
  if (n_sel >= n_sc)
    written = ordered_compact<NT, V>(n_sc, wcnt, [&](int, int&) { return true; },
                                     [&](int r, int m, int) {
                                       if (r < n_keep - 1) out[r] = m;
                                     });
  else if (n_sel > 0)
    written = blk_cut_passes<NT>(br, n_sc, n_sel, out);
  written = min(written, n_keep - 1);
  if (tid == 0) out[written] = own;
  for (int t = written + 1 + tid; t < n_keep; t += NT) out[t] = -1;
}

// Block keep of long prefill-shaped rows (up to BLK_LONG_MAXB blocks): the result of
// blk_select_kernel from two reads of the row instead of about eight.  The first counts
// the keys per coarse bin (coarse_bin64, monotone in the score) and finds the bin b*
// holding the cut; the second marks the blocks of higher bins in an LDS bitmap of
// positions and gathers b*'s members (key, position) into LDS, where the exact cut, the
// ties it keeps (lowest positions) and the bitmap's remaining bits are settled; the
// bitmap is then written out in position order.  Rows of up to MAXB blocks; a row whose
// b* holds more than MCAP members (heavy ties) takes blk_cut_passes instead.
// Measured on MI355X: rows of 1024 blocks are faster with blk_select_kernel (its
// passes hit the cache), rows of 4K-16K blocks with the 256-thread form (three
// workgroups per compute unit), longer rows with the 1024-thread form.
constexpr int BLK_LONG_MAXB = 131072;
constexpr int BLK_MED_MIN = 4096, BLK_MED_MAXB = 16384;
template <int NT, int MAXB, int MCAP>
__global__ __launch_bounds__(NT) void blk_select_long_kernel(const long long* __restrict__ bscores, long long ld,
                                                             const int32_t* __restrict__ q_pos, int n_blocks,
                                                             int bs, int n_keep, int32_t* __restrict__ kept,
    const int32_t* __restrict__ rstate) {
  constexpr int V = 8, MC = MCAP / NT, NWD = MAXB / 32;
  static_assert(MCAP % NT == 0 && NBINS % NT == 0 && MC <= 32, "whole member and bin ranges per thread");
  __shared__ int hist[NBINS];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ unsigned long long mkey[MCAP];
  __shared__ int mpos[MCAP];
  __shared__ int scan_tmp[NT / 64 + 1], sh[8], mcnt;
  __shared__ unsigned long long shu[2];
  const long long row = blockIdx.x;
  if (rstate != nullptr && rstate[row] == 0) return;  // kept from its list
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = q_pos[row];
  int32_t* out = kept + row * (long long)n_keep;
  if (p < 0) {
    for (int t = tid; t < n_keep; t += NT) out[t] = -1;
    return;
  }
  const int own = p / bs;
  const int n_sc = min(own, n_blocks);  // scored earlier blocks
  const int n_sel = min(n_keep - 1, n_sc);
  const long long* br = bscores + row * ld;
  int written;
  if (n_sel >= n_sc) {
    for (int m = tid; m < n_sc; m += NT) out[m] = m;
    written = n_sc;
  } else {
    for (int t = tid; t < NBINS; t += NT) hist[t] = 0;
    __syncthreads();
    for (int base = 0; base < n_sc; base += V * NT) {
      long long s[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int m = base + v * NT + tid;
        s[v] = m < n_sc ? br[m] : 0ll;
      }
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (base + v * NT + tid < n_sc) atomicAdd(&hist[coarse_bin64(s[v])], 1);
    }
    __syncthreads();
    find_cut_bin<NT>(hist, n_sel, scan_tmp, sh);
    const int bstar = sh[4], cnt = sh[6];
    const int need = n_sel - sh[5];  // 1 .. cnt of b*'s members are kept
    if (cnt <= MCAP) {
      const int nwd = (n_sc + 31) >> 5;
      for (int t = tid; t < nwd; t += NT) eqm[t] = 0u;
      if (tid == 0) mcnt = 0;
      __syncthreads();
      for (int base = 0; base < n_sc; base += V * NT) {
        long long s[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int m = base + v * NT + tid;
          s[v] = m < n_sc ? br[m] : 0ll;
        }
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int m = base + v * NT + tid;
          const int b = m < n_sc ? coarse_bin64(s[v]) : -1;
          // the wave's 64 positions are two whole bitmap words, each written once
          const unsigned long long gt = __ballot(b > bstar);
          const int w0 = (base + v * NT + wave * 64) >> 5;
          if (lane < 2 && w0 + lane < nwd) bm[w0 + lane] = (unsigned)(gt >> (32 * lane));
          const unsigned long long in = __ballot(b == bstar);
          if (in != 0ull) {
            int slot0 = 0;
            if (lane == 0) slot0 = atomicAdd(&mcnt, __popcll(in));
            slot0 = __shfl(slot0, 0);
            if (b == bstar) {
              const int j = slot0 + lanes_below(in);
              mkey[j] = (unsigned long long)s[v] ^ 0x8000000000000000ull;
              mpos[j] = m;
            }
          }
        }
      }
      __syncthreads();
      unsigned long long key[MC];
      int pos[MC];
      unsigned vmask = 0u;
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        const int j = c * NT + tid;
        key[c] = j < cnt ? mkey[j] : 0ull;
        pos[c] = j < cnt ? mpos[j] : 0;
        vmask |= (j < cnt ? 1u : 0u) << c;
      }
      int need_eq;
      const unsigned long long T = radix_cut64<NT, MC>(key, vmask, need, hist, scan_tmp, sh, shu, &need_eq);
#pragma unroll
      for (int c = 0; c < MC; ++c) {
        if (!((vmask >> c) & 1u)) continue;
        if (key[c] > T) atomicOr(&bm[pos[c] >> 5], 1u << (pos[c] & 31));
        else if (key[c] == T) atomicOr(&eqm[pos[c] >> 5], 1u << (pos[c] & 31));
      }
      __syncthreads();
      keep_first_ties<NT>(bm, eqm, nwd, need_eq, scan_tmp);
      written = emit_marked<NT>(bm, nwd, scan_tmp, [&](int r, int q) {
        if (r < n_sel) out[r] = q;
      });
    } else {
      written = blk_cut_passes<NT>(br, n_sc, n_sel, out);
    }
  }
  written = min(written, n_keep - 1);
  if (tid == 0) out[written] = own;
  for (int t = written + 1 + tid; t < n_keep; t += NT) out[t] = -1;
}

// Block keep of rows with many blocks and one workgroup each (decode): the same result
// as blk_select_kernel, with the row's scores held in registers (thread t: blocks
// t, t + NT, ..., at most C of them) instead of re-read per pass: the cut (radix_cut64)
// and, in block order, the blocks with a higher key and the first ones equal to the cut.
template <int NT, int C>
__global__ __launch_bounds__(NT) void blk_keep_rows_kernel(const long long* __restrict__ bscores, long long ld,
                                                           const int32_t* __restrict__ q_pos, int n_blocks, int bs,
                                                           int n_keep, int32_t* __restrict__ kept,
    const int32_t* __restrict__ rstate) {
  constexpr int NW = NT / 64, NWD = NT * C / 32;
  __shared__ int hist[2048];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ int scan_tmp[NW + 1], sh[2];
  __shared__ unsigned long long shu[2];
  const long long row = blockIdx.x;
  if (rstate != nullptr && rstate[row] == 0) return;  // kept from its list
  const int tid = threadIdx.x;
  const int p = q_pos[row];
  int32_t* out = kept + row * (long long)n_keep;
  if (p < 0) {
    for (int t = tid; t < n_keep; t += NT) out[t] = -1;
    return;
  }
  const int own = p / bs;
  const int n_sc = min(own, n_blocks);  // scored earlier blocks
  const int n_sel = min(n_keep - 1, n_sc);
  const long long* br = bscores + row * ld;
  int written;
  if (n_sel >= n_sc) {
    for (int m = tid; m < n_sc; m += NT) out[m] = m;
    written = n_sc;
  } else {
    unsigned long long key[C];
    unsigned vmask = 0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int m = c * NT + tid;
      key[c] = m < n_sc ? (unsigned long long)br[m] ^ 0x8000000000000000ull : 0ull;
      vmask |= (m < n_sc ? 1u : 0u) << c;
    }
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, n_sel, hist, scan_tmp, sh, shu, &need_eq);
    mark_kept64<NT, C>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
    written = emit_marked<NT>(bm, NWD, scan_tmp, [&](int r, int pos) {
      if (r < n_keep - 1) out[r] = pos;
    });
  }
  written = min(written, n_keep - 1);
  if (tid == 0) out[written] = own;
  for (int t = written + 1 + tid; t < n_keep; t += NT) out[t] = -1;
}

// Block keep of decode-shaped rows from the scoring workgroups' candidates (BlkCand):
// every span holding scored blocks left its best min(n_keep - 1, its blocks) in block
// order, so their concatenation is in block order and holds every block the row keeps;
// the row's cut over it (at most NT * C entries, in registers) is the row's.
template <int NT, int C>
__global__ __launch_bounds__(NT) void blk_keep_merge_kernel(const int32_t* __restrict__ q_pos, int n_blocks, int bs,
                                                            int n_keep, BlkCand cand, int32_t* __restrict__ kept) {
  constexpr int NW = NT / 64, NWD = NT * C / 32;
  constexpr int MAX_SPANS = 256;
  static_assert(NT > MAX_SPANS, "one thread per span");
  __shared__ int hist[2048];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ int blk_s[NT * C];
  __shared__ int off_s[MAX_SPANS + 1];
  __shared__ int scan_tmp[NW + 1], sh[2];
  __shared__ unsigned long long shu[2];
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
  const int n_sel = min(n_keep - 1, n_sc);
  int written;
  if (n_sel >= n_sc) {
    for (int m = tid; m < n_sc; m += NT) out[m] = m;
    written = n_sc;
  } else {
    const int S = (n_sc + cand.span - 1) / cand.span;  // spans with scored blocks (each wrote its list)
    const long long rs = row * cand.spans;
    // list offsets: the counts load in parallel, one thread per span, then one scan
    const int my_cnt = tid < S ? cand.cnt[rs + tid] : 0;
    int total;
    const int my_off = block_exclusive_scan<NT>(my_cnt, scan_tmp, &total);
    if (tid <= S) off_s[tid] = tid < S ? my_off : total;
    __syncthreads();
    unsigned long long key[C];
    unsigned vmask = 0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = c * NT + tid;
      key[c] = 0ull;
      if (e < total) {
        int lo = 0, hi = S;  // the span whose list holds entry e: off_s[lo] <= e < off_s[lo + 1]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (off_s[mid] <= e) lo = mid;
          else hi = mid;
        }
        const long long at = (rs + lo) * cand.cap + (e - off_s[lo]);
        key[c] = (unsigned long long)cand.key[at] ^ 0x8000000000000000ull;
        blk_s[e] = cand.blk[at];
        vmask |= 1u << c;
      }
    }
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, n_sel, hist, scan_tmp, sh, shu, &need_eq);
    mark_kept64<NT, C>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
    written = emit_marked<NT>(bm, NWD, scan_tmp, [&](int r, int pos) {
      if (r < n_keep - 1) out[r] = blk_s[pos];
    });
  }
  written = min(written, n_keep - 1);
  if (tid == 0) out[written] = own;
  for (int t = written + 1 + tid; t < n_keep; t += NT) out[t] = -1;
}

}  // namespace

size_t topk_ws_bytes(long long rows, int L_max) {
  if (rows == 0 || rows > 512 || L_max < 4 * SEG) return 0;
  const long long n_seg = (L_max + SEG - 1) / SEG;
  if (n_seg > 1024) return 0;
  return (size_t)rows * (size_t)SegWs::row_ints_for(n_seg) * sizeof(int);
}

static bool split_rows(const TopkArgs& a, SegWs* w) {
  const long long rows = (long long)a.B * a.n_q;
  const size_t need = topk_ws_bytes(rows, a.L_max);
  if (a.kept != nullptr || need == 0 || a.ws == nullptr || a.ws_bytes < need) return false;
  w->base = static_cast<int*>(a.ws);
  w->n_seg = (a.L_max + SEG - 1) / SEG;
  return true;
}

// spans per row of the decode selection: about DEC_WGS workgroups in all, spans of at
// least DEC_SPAN_MIN keys, and as many as a span of at most DEC_SPAN_MAX keys needs
static long long dec_parts(long long rows, int L_max) {
  const long long by_lds = (L_max + (DEC_SPAN_MAX - 64)) / (DEC_SPAN_MAX - 63);
  const long long by_fill = (DEC_WGS + rows - 1) / rows;
  const long long by_size = std::max<long long>(1, L_max / DEC_SPAN_MIN);
  return std::max(by_lds, std::min(by_fill, by_size));
}

bool dec_sel_layout(long long rows, int L_max, int k, DecLayout* out) {
  if (rows < 1 || rows > 65535 || L_max < 1 || k < 1) return false;
  const long long parts = dec_parts(rows, L_max);
  if (parts > DEC_MAX_PARTS) return false;
  // a list holds at least min(span, k) entries, plus the rest of the bin that completes it
  out->parts = (int)parts;
  out->lcap = (int)std::min<long long>((2ll * k + 3) / 4 * 4, DEC_SPAN_MAX);
  out->rec_ints = DecWs::rec_ints_for(out->lcap);
  return true;
}

size_t dec_sel_ws_bytes(long long rows, int L_max, int k) {
  DecLayout d;
  if (!dec_sel_layout(rows, L_max, k, &d)) return 0;
  // records of a chunk of r <= rows rows: r * parts(r) <= r * max(by_lds, min(by_fill(r),
  // by_size)), and r * by_fill(r) <= r + DEC_WGS - 1
  const long long by_lds = (L_max + (DEC_SPAN_MAX - 64)) / (DEC_SPAN_MAX - 63);
  const long long by_size = std::max<long long>(1, L_max / DEC_SPAN_MIN);
  const long long recs = std::max(rows * by_lds, std::min(rows + DEC_WGS - 1, rows * by_size));
  return (size_t)recs * (size_t)d.rec_ints * sizeof(int);
}

static bool dec_rows(const TopkArgs& a, DecWs* w) {
  const long long rows = (long long)a.B * a.n_q;
  DecLayout d;
  if (a.kept != nullptr || a.ws == nullptr || !dec_sel_layout(rows, a.L_max, a.k, &d) ||
      a.ws_bytes < (size_t)rows * d.parts * (size_t)d.rec_ints * sizeof(int))
    return false;
  w->base = static_cast<int*>(a.ws);
  w->rec_ints = d.rec_ints;
  w->parts = d.parts;
  w->lcap = d.lcap;
  return true;
}

template <bool KEPT>
static hipError_t launch_topk_t(const TopkArgs& a, hipStream_t st, long long rows) {
  if (!KEPT && a.hist_ready) {
    // the decode indexer left each span's histogram and list: one kernel
    DecWs d;
    if (!dec_rows(a, &d)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((topk_list_finish_kernel<1024>), dim3((unsigned)rows), dim3(1024), 0, st,
                       const_cast<int32_t*>(a.scores), a.ld, a.q_pos, a.L_max, a.k, d, a.idx, a.count, a.n_q,
                       a.pages);
    return hipGetLastError();
  }
  SegWs w;
  if (!KEPT && a.row_state == nullptr && a.pages.page_table == nullptr && split_rows(a, &w)) {
    // several workgroups per row: histogram and candidate compaction split over segments
    const dim3 grid((unsigned)w.n_seg, (unsigned)rows);
    hipLaunchKernelGGL(topk_seg_zero_kernel, dim3(8, (unsigned)rows), dim3(256), 0, st, w.base, w.row_ints(), rows);
    hipLaunchKernelGGL((topk_seg_hist_kernel<256, KEPT>), grid, dim3(256), 0, st, a.scores, a.ld, a.q_pos, a.kept,
                       a.block_size, a.n_keep, a.L_max, a.k, w);
    hipLaunchKernelGGL((topk_seg_select_kernel<256>), grid, dim3(256), 0, st, a.scores, a.ld, a.q_pos, a.L_max,
                       a.k, w);
    hipLaunchKernelGGL((topk_seg_finish_kernel<256, KEPT>), dim3((unsigned)rows), dim3(256), 0, st, a.scores,
                       a.ld, a.q_pos, a.kept, a.block_size, a.n_keep, a.L_max, a.k, w, a.idx, a.count);
    return hipGetLastError();
  }
  if (rows <= 1024 && a.L_max >= 16384) {
    hipLaunchKernelGGL((topk_kernel<1024, KEPT>), dim3((unsigned)rows), dim3(1024), 0, st, a.scores, a.ld, a.q_pos,
                       a.kept, a.block_size, a.n_keep, a.L_max, a.k, a.idx, a.count, a.row_state, a.n_q, a.pages);
  } else {
    hipLaunchKernelGGL((topk_kernel<256, KEPT>), dim3((unsigned)rows), dim3(256), 0, st, a.scores, a.ld, a.q_pos,
                       a.kept, a.block_size, a.n_keep, a.L_max, a.k, a.idx, a.count, a.row_state, a.n_q, a.pages);
  }
  return hipGetLastError();
}

hipError_t launch_thresholds(const int32_t* samp, long long ld_s, const int32_t* q_pos, long long rows, int L_max,
                             int k, int stride, int mode, const ThrArgs& t, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > THR_MAX_K || t.cap != thr_cap(k) || t.row_min < t.cap || L_max > THR_MAX_L || stride < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(thr_kernel<256>, dim3((unsigned)rows), dim3(256), 0, st, samp, ld_s, q_pos, L_max, k, stride,
                     mode, t);
  return hipGetLastError();
}

hipError_t launch_list_topk(const int32_t* q_pos, long long rows, int L_max, int k, const ThrArgs& t,
                            int32_t* idx, int32_t* count, int n_q, const Pages& pg, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > THR_MAX_K || t.cap != thr_cap(k) || L_max > THR_MAX_L) return hipErrorInvalidValue;
  constexpr int NT = 256, J = 4 * THR_MAX_K / (4 * NT);  // J quads a thread hold the longest list
  const size_t dyn = (size_t)max(NBINS, (L_max + 31) / 32) * sizeof(int);
  hipLaunchKernelGGL((list_topk_kernel<NT, J>), dim3((unsigned)rows), dim3(NT), dyn, st, q_pos, L_max, k, t, idx,
                     count, n_q, pg);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  return a.kept != nullptr ? launch_topk_t<true>(a, st, rows) : launch_topk_t<false>(a, st, rows);
}

// Threshold of each block row for the thresholded keep (one workgroup per row).  A row
// with at most row_min scored blocks (or no position) keeps the score table (state 1).
// Otherwise its threshold is the t-th best of its m sampled scores (blocks 0, stride,
// 2 stride, ... below its own block), t = ceil(2 n_sel m / n_sc) (at most m), so about
// 2 n_sel of its blocks are expected to reach it; the keep stays exact whatever the
// sample shows (lists that fall short or overflow take the table).  The m samples sit
// in registers, C per thread (the launcher checks m <= NT * C).
// It also clears the fallback tile list (row 0) and its row's tile mark (first row of a tile).
template <int NT, int C>
__global__ __launch_bounds__(NT) void blk_thr_kernel(const long long* __restrict__ samp, long long ld_s,
                                                     const int32_t* __restrict__ q_pos, int n_q, int n_blocks,
                                                     int bs, int n_keep, int stride, int row_min, int mode,
                                                     BlkThr t) {
  __shared__ int hist[2048];
  __shared__ int scan_tmp[NT / 64 + 1], sh[8];
  __shared__ unsigned long long shu[2];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const int i = (int)(row % n_q);
    if (i % BLK_THR_QT == 0)
      t.tflag[(row / n_q) * ((n_q + BLK_THR_QT - 1) / BLK_THR_QT) + i / BLK_THR_QT] = 0;
    if (row == 0) *t.tcnt = 0;
  }
  const int p = q_pos[row];
  const int n_sc = p >= 0 ? min(p / bs, n_blocks) : 0;  // scored blocks
  if (p < 0 || n_sc <= row_min) {
    if (tid == 0) {
      t.theta[row] = LLONG_MIN;
      t.rstate[row] = 1;
      t.cnt[row] = 0;
    }
    return;
  }
  const int n_sel = min(n_keep - 1, n_sc);
  long long th;
  if (mode == 1) {
    th = LLONG_MAX;
  } else if (mode == 2) {
    th = LLONG_MIN;
  } else {
    const int m = (n_sc + stride - 1) / stride;
    const long long tt = (2LL * n_sel * m + n_sc - 1) / n_sc;
    const int need = (int)min<long long>(m, max<long long>(1, tt));
    const long long* sr = samp + row * ld_s;
    unsigned long long key[C];
    unsigned vmask = 0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = c * NT + tid;
      key[c] = j < m ? (unsigned long long)sr[j] ^ 0x8000000000000000ull : 0ull;
      vmask |= (j < m ? 1u : 0u) << c;
    }
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, need, hist, scan_tmp, sh, shu, &need_eq);
    th = (long long)(T ^ 0x8000000000000000ull);
  }
  if (tid == 0) {
    t.theta[row] = th;
    t.rstate[row] = 0;
    t.cnt[row] = 0;
  }
}

// Exact keep of a list row (one workgroup per row, rows in state 0): every scored
// block whose score reaches the row's threshold is in its list, and there are at least
// n_sel of them, so the row's best n_sel blocks by (score desc, block asc) are the
// list's.  The list (at most NT * C entries) sits in registers: the cut over it
// (radix_cut64), the blocks above the cut and the lowest-numbered ones equal to it
// (an LDS bitmap of block positions), written ascending, then the own block and -1s.
// A list that fell short of n_sel or overflowed marks its row (state 2) for the table.
template <int NT, int C>
__global__ __launch_bounds__(NT) void blk_list_keep_kernel(const int32_t* __restrict__ q_pos, int n_q, int n_blocks,
                                                           int bs, int n_keep, BlkThr t,
                                                           int32_t* __restrict__ kept) {
  constexpr int NWD = BLK_THR_MAX_B / 32;
  __shared__ int hist[2048];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ int scan_tmp[NT / 64 + 1], sh[8];
  __shared__ unsigned long long shu[2];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  if (t.rstate[row] != 0) return;
  const int own = q_pos[row] / bs;  // a list row has a position and more than row_min scored blocks
  const int n_sc = min(own, n_blocks);
  const int n_sel = min(n_keep - 1, n_sc);
  const int c = t.cnt[row];
  if (c < n_sel || c > t.cap) {
    if (tid == 0) {
      t.rstate[row] = 2;
      // the row's tile, listed once for the fallback scoring
      const int tile = (int)((row / n_q) * ((n_q + BLK_THR_QT - 1) / BLK_THR_QT) + (row % n_q) / BLK_THR_QT);
      if (atomicExch(&t.tflag[tile], 1) == 0) t.tlist[atomicAdd(t.tcnt, 1)] = tile;
    }
    return;
  }
  const int32_t* lb = t.lblk + row * t.cap;
  const long long* ls = t.lscore + row * t.cap;
  unsigned long long key[C];
  int pos[C];
  unsigned vmask = 0u;
#pragma unroll
  for (int cc = 0; cc < C; ++cc) {
    const int j = cc * NT + tid;
    key[cc] = j < c ? (unsigned long long)ls[j] ^ 0x8000000000000000ull : 0ull;
    pos[cc] = j < c ? lb[j] : 0;
    vmask |= (j < c ? 1u : 0u) << cc;
  }
  int need_eq;
  const unsigned long long T = radix_cut64<NT, C>(key, vmask, n_sel, hist, scan_tmp, sh, shu, &need_eq);
  const int nwd = (n_sc + 31) >> 5;
  for (int wd = tid; wd < nwd; wd += NT) {
    bm[wd] = 0u;
    eqm[wd] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int cc = 0; cc < C; ++cc) {
    if (!((vmask >> cc) & 1u)) continue;
    if (key[cc] > T) atomicOr(&bm[pos[cc] >> 5], 1u << (pos[cc] & 31));
    else if (key[cc] == T) atomicOr(&eqm[pos[cc] >> 5], 1u << (pos[cc] & 31));
  }
  __syncthreads();
  keep_first_ties<NT>(bm, eqm, nwd, need_eq, scan_tmp);
  int32_t* out = kept + row * (long long)n_keep;
  const int written = emit_marked<NT>(bm, nwd, scan_tmp, [&](int r, int q) {
    if (r < n_sel) out[r] = q;
  });
  const int wr = min(written, n_sel);
  if (tid == 0) out[wr] = own;
  for (int tt = wr + 1 + tid; tt < n_keep; tt += NT) out[tt] = -1;
}

hipError_t launch_blk_thresholds(const long long* samp, long long ld_s, const int32_t* q_pos, int B, int n_q,
                                 int n_blocks, int bs, int n_keep, int stride, int row_min, int mode,
                                 const BlkThr& t, hipStream_t st) {
  const long long rows = (long long)B * n_q;
  if (rows == 0) return hipSuccess;
  constexpr int NT = 256, C = BLK_THR_MAX_SAMPLES / 256;
  if (samp == nullptr || t.theta == nullptr || t.rstate == nullptr || t.cnt == nullptr || t.tflag == nullptr ||
      t.tcnt == nullptr || stride < 1 || bs < 1 || n_keep < 2 || mode < 0 || mode > 2 ||
      (long long)(n_blocks + stride - 1) / stride > (long long)NT * C || ld_s < (n_blocks + stride - 1) / stride)
    return hipErrorInvalidValue;
  // samples per thread: as few registers as the longest row needs
  const int m_max = (n_blocks + stride - 1) / stride;
  if (m_max <= NT * 8)
    hipLaunchKernelGGL((blk_thr_kernel<NT, 8>), dim3((unsigned)rows), dim3(NT), 0, st, samp, ld_s, q_pos, n_q,
                       n_blocks, bs, n_keep, stride, row_min, mode, t);
  else if (m_max <= NT * 16)
    hipLaunchKernelGGL((blk_thr_kernel<NT, 16>), dim3((unsigned)rows), dim3(NT), 0, st, samp, ld_s, q_pos, n_q,
                       n_blocks, bs, n_keep, stride, row_min, mode, t);
  else
    hipLaunchKernelGGL((blk_thr_kernel<NT, C>), dim3((unsigned)rows), dim3(NT), 0, st, samp, ld_s, q_pos, n_q,
                       n_blocks, bs, n_keep, stride, row_min, mode, t);
  return hipGetLastError();
}

hipError_t launch_blk_list_keep(const int32_t* q_pos, int B, int n_q, int n_blocks, int bs, int n_keep,
                                const BlkThr& t, int32_t* kept, hipStream_t st) {
  const long long rows = (long long)B * n_q;
  if (rows == 0) return hipSuccess;
  constexpr int NT = 256;
  if (t.lblk == nullptr || t.lscore == nullptr || t.cap < 1 || t.tflag == nullptr || t.tlist == nullptr ||
      t.tcnt == nullptr || n_blocks > BLK_THR_MAX_B || n_keep < 2 || kept == nullptr)
    return hipErrorInvalidValue;
  if (t.cap <= NT * 8)
    hipLaunchKernelGGL((blk_list_keep_kernel<NT, 8>), dim3((unsigned)rows), dim3(NT), 0, st, q_pos, n_q, n_blocks,
                       bs, n_keep, t, kept);
  else if (t.cap <= NT * 32)
    hipLaunchKernelGGL((blk_list_keep_kernel<NT, 32>), dim3((unsigned)rows), dim3(NT), 0, st, q_pos, n_q,
                       n_blocks, bs, n_keep, t, kept);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Pooled blocks: the index list of a query is every key of its kept blocks that it
// may see, idx[r] = kept[r / bs] * bs + r % bs if that block is kept and the key is
// <= the query's position, else -1.  kept is ascending with the own block last, so
// the valid keys form a prefix in ascending order; count = their number.
template <int NT>
__global__ __launch_bounds__(NT) void expand_kernel(const int32_t* __restrict__ kept, const int32_t* __restrict__ q_pos,
                                                    int bs, int n_keep, int k, int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ count, Pages pg, int n_q) {
  __shared__ int scan_tmp[NT / 64 + 1];
  const long long row = blockIdx.x;
  const int p = q_pos[row];
  const int32_t* kr = kept + row * (long long)n_keep;
  int32_t* out = idx + row * (long long)k;
  // paged caches: the list holds pool rows (row / n_q is the row's sequence)
  const int32_t* pt = pg.page_table != nullptr ? pg.page_table + (row / n_q) * pg.max_pages : nullptr;
  const int pmask = (1 << pg.page_log2) - 1;
  int n = 0;
  for (int r = threadIdx.x; r < k; r += NT) {
    const int blk = r / bs < n_keep ? kr[r / bs] : -1;
    const int key = blk * bs + r % bs;
    const bool ok = blk >= 0 && key <= p;
    int v = ok ? key : -1;
    if (ok && pt != nullptr) v = (min(max(pt[key >> pg.page_log2], 0), pg.n_pages - 1) << pg.page_log2) | (key & pmask);
    out[r] = v;
    n += ok ? 1 : 0;
  }
  if (count != nullptr) {
    int tot;
    block_exclusive_scan<NT>(n, scan_tmp, &tot);
    if (threadIdx.x == 0) count[row] = tot;
  }
}

hipError_t launch_expand(const int32_t* kept, const int32_t* q_pos, long long rows, int bs, int n_keep, int k,
                         int32_t* idx, int32_t* count, hipStream_t st, const Pages& pg, int n_q) {
  if (rows == 0) return hipSuccess;
  if (bs < 1 || n_keep < 1 || k < 1 || n_q < 1) return hipErrorInvalidValue;
  if (pg.page_table != nullptr && (pg.page_log2 < 6 || pg.page_log2 > 30 || pg.n_pages < 1)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_kernel<256>, dim3((unsigned)rows), dim3(256), 0, st, kept, q_pos, bs, n_keep, k, idx,
                     count, pg, n_q);
  return hipGetLastError();
}

size_t kidx_interleave_bytes(int B, int L_max, int d_I) {
  return (size_t)B * (size_t)((L_max + 63) / 64) * 64 * (size_t)d_I;
}

hipError_t launch_kidx_interleave(const int8_t* k_idx, int B, int L_max, int d_I, const Pages& pg, int8_t* out,
                                  hipStream_t st) {
  if (B < 1 || L_max < 1 || (d_I != 64 && d_I != 128) || !k_idx || !out) return hipErrorInvalidValue;
  if (pg.page_table != nullptr &&
      (pg.page_log2 < 6 || pg.page_log2 > 30 || pg.n_pages < 1 || (long long)pg.max_pages << pg.page_log2 != L_max))
    return hipErrorInvalidValue;
  const long long n_grp = (L_max + 63) / 64;
  const long long total = (long long)B * n_grp * 64 * (d_I / 16);
  const unsigned grid = (unsigned)std::min<long long>((total + 255) / 256, 16LL * device_cus());
  if (d_I == 128)
    hipLaunchKernelGGL(kidx_interleave_kernel<128>, dim3(grid), dim3(256), 0, st, k_idx, L_max, n_grp, total, pg,
                       reinterpret_cast<v4i*>(out));
  else
    hipLaunchKernelGGL(kidx_interleave_kernel<64>, dim3(grid), dim3(256), 0, st, k_idx, L_max, n_grp, total, pg,
                       reinterpret_cast<v4i*>(out));
  return hipGetLastError();
}

hipError_t launch_kept_select(const IdxArgs& a, int k, int32_t* idx, int32_t* count, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  if (a.kept == nullptr || a.block_size < 1 || a.n_keep < 1 || a.n_keep > 256 ||
      (long long)a.n_keep * a.block_size > KSEL_SLOTS || k < 1 || (a.d_I != 64 && a.d_I != 128) || a.H_I < 1 ||
      a.H_I > 64)
    return hipErrorInvalidValue;
  if (a.pages.page_table != nullptr &&
      (a.pages.page_log2 < 6 || a.pages.page_log2 > 30 || a.pages.n_pages < 1 ||
       (long long)a.pages.max_pages << a.pages.page_log2 != a.L_max))
    return hipErrorInvalidValue;
  const int mt = (a.H_I + 15) / 16;
  if (a.d_I == 128) {
    switch (mt) {
      case 1: return launch_kept_select_t<128, 1>(a, k, idx, count, st);
      case 2: return launch_kept_select_t<128, 2>(a, k, idx, count, st);
      case 3: return launch_kept_select_t<128, 3>(a, k, idx, count, st);
      default: return launch_kept_select_t<128, 4>(a, k, idx, count, st);
    }
  }
  switch (mt) {
    case 1: return launch_kept_select_t<64, 1>(a, k, idx, count, st);
    case 2: return launch_kept_select_t<64, 2>(a, k, idx, count, st);
    case 3: return launch_kept_select_t<64, 3>(a, k, idx, count, st);
    default: return launch_kept_select_t<64, 4>(a, k, idx, count, st);
  }
}

hipError_t launch_block_select(const BlkSelArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  if (a.cand.key != nullptr) {
    // decode-shaped rows whose scoring left span candidates
    if (a.cand.spans > 256 || (long long)a.cand.spans * a.cand.cap > 8 * 1024 || a.cand.cap != a.n_keep - 1)
      return hipErrorInvalidValue;
    hipLaunchKernelGGL((blk_keep_merge_kernel<1024, 8>), dim3((unsigned)rows), dim3(1024), 0, st, a.q_pos,
                       a.n_blocks, a.block_size, a.n_keep, a.cand, a.kept);
    return hipGetLastError();
  }
  if (a.n_q < 8 && a.n_blocks > 4096 && a.n_blocks <= 1024 * 32) {
    // few long rows (decode): the row's scores in registers of one workgroup
    hipLaunchKernelGGL((blk_keep_rows_kernel<1024, 32>), dim3((unsigned)rows), dim3(1024), 0, st, a.bscores, a.ld,
                       a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept, a.rstate);
    return hipGetLastError();
  }
  if (a.n_blocks > 4096 && a.n_blocks <= 512 * 16) {
    // prefill-shaped rows of up to 8192 blocks: the row in registers, read once
    // (prefill_32k_pool4's keep 0.82 -> 0.67 ms against the two-read kernel below)
    hipLaunchKernelGGL((blk_keep_rows_kernel<512, 16>), dim3((unsigned)rows), dim3(512), 0, st, a.bscores, a.ld,
                       a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept, a.rstate);
    return hipGetLastError();
  }
  if (a.n_blocks > BLK_MED_MAXB && a.n_blocks <= BLK_LONG_MAXB) {
    // long prefill-shaped rows: two reads of each row
    hipLaunchKernelGGL((blk_select_long_kernel<1024, BLK_LONG_MAXB, 4096>), dim3((unsigned)rows), dim3(1024), 0, st,
                       a.bscores, a.ld, a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept, a.rstate);
    return hipGetLastError();
  }
  if (a.n_blocks > BLK_MED_MIN && a.n_blocks <= BLK_MED_MAXB) {
    hipLaunchKernelGGL((blk_select_long_kernel<256, BLK_MED_MAXB, 1024>), dim3((unsigned)rows), dim3(256), 0, st,
                       a.bscores, a.ld, a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept, a.rstate);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(blk_select_kernel<256>, dim3((unsigned)rows), dim3(256), 0, st, a.bscores, a.ld,
                     a.q_pos, a.n_blocks, a.block_size, a.n_keep, a.kept, a.rstate);
  return hipGetLastError();
}

}  // namespace lsa
