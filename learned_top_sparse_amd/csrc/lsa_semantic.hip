// lsa_semantic.hip -- flat semantic search: Ward clustering of cluster blocks into a
// bucket cache, centroid scoring, exact top-p of the buckets and their expansion into
// the index lists ("Latent Sparse Attention (LSA)" §3.1 "Semantic Clustering", §3.2
// "Semantic Search", App. F.1 "Kernels").
//
// Floating point takes integer decisions here (which buckets merge, which are kept),
// so this file is compiled with -ffp-contract=off: every sum and product is rounded on
// its own, in the order written, and sums over the 64 index dimensions run d = 0, 1,
// ...  The one fused multiply-add is explicit and adds exact products (bf16 x bf16 is
// exact in fp32), so it rounds like the separate add.  Division and square root are
// the correctly rounded ones.
//
// Bucket cache of sequence b, cluster block t (m <= 64 buckets per block, listed by the
// lowest pool key each holds):
//   centroids bf16 [B][NB][8][64][8]: dims 8c..8c+7 of bucket slot s at [c][s][0..7]
//     (slots m..63 zero), so a wave reads one dim group of all 64 slots as 1 KB;
//   table int32 [B][NB][n_cluster]: key positions, bucket after bucket, ascending
//     within a bucket;
//   offsets int32 [B][NB][m + 1]: bucket starts in the table (offsets[m] = n_cluster).
#include <hip/hip_runtime.h>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "lsa_select.h"

namespace lsa {
namespace {

constexpr int SEM_D = 64;        // index dimension
constexpr int SEM_NPK = 128;     // pool keys per cluster block, at most
constexpr int SEM_SLOTS = 64;    // bucket slots per block in the centroid layout
constexpr int SEL_NT = 512;      // threads of the selection workgroup

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, nearest with ties to even (finite inputs)
__device__ __forceinline__ unsigned to_bf16(float x) {
  const unsigned u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// order-keeping unsigned image of an fp32 score (-0 just below +0)
__device__ __forceinline__ unsigned order_key(float s) {
  const unsigned u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void unpack8(uint4 v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Where a sequence's cluster block lives in the bucket cache, and where its logical key
// lives in the index-key / K / V storage: identity for contiguous caches, through a
// block table and a page table for pooled ones (ids clamped into their pools).
struct SemPaging {
  const int* bt;     // [B][NB] cache slot of each block, or null: slot b * NB + t
  int n_bslots;
  const int* pt;     // [B][max_pages] pool page of each page of keys, or null: contiguous
  int plog2, max_pages;
  long long n_pages;
  __device__ __forceinline__ long long slot(int b, int NB, int blk) const {
    if (!bt) return (long long)b * NB + blk;
    int v = bt[(long long)b * NB + blk];
    v = v < 0 ? 0 : (v >= n_bslots ? n_bslots - 1 : v);
    return v;
  }
  // storage row of logical key j of sequence b (rows of L_max per sequence if contiguous)
  __device__ __forceinline__ long long row(int b, long long L_max, int j) const {
    if (!pt) return (long long)b * L_max + j;
    int pi = j >> plog2;
    pi = pi < max_pages ? pi : max_pages - 1;  // positions past the pages stay in the table
    long long pg = pt[(long long)b * max_pages + pi];
    pg = pg < 0 ? 0 : (pg >= n_pages ? n_pages - 1 : pg);
    return (pg << plog2) | (j & ((1 << plog2) - 1));
  }
  // what the index list holds for logical key j: the key itself if contiguous, its pool row if paged
  __device__ __forceinline__ int list_entry(int b, int j) const { return pt ? (int)row(b, 0, j) : j; }
};

// ---------------------------------------------------------------------------------
// Clustering: one 1024-thread workgroup per (cluster block, sequence), 8 threads per
// pool key / bucket row.  The block's pool keys (sums of its normalised keys), the
// bucket sums and the Ward cost of every pair stay in LDS for all merge rounds; only
// the costs against merged buckets are recomputed after a round.

struct SemGeom {
  int n_cluster, n_pool, npk, m, cap;  // cap: size cap in pool keys
};

// Ward's cost of buckets a, b: |n_b S_a - n_a S_b|^2 / (n_a n_b (n_a + n_b)).  Four
// costs of bucket a at once, each summed d = 0, 1, ... on its own chain, so the order
// of every rounding is that of one cost at a time.
__device__ __forceinline__ void ward_cost4(const float (*S)[SEM_D + 1], int a, float na, const int* bb,
                                           const float* nb, float* out) {
  float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int d = 0; d < SEM_D; ++d) {
    const float sad = S[a][d];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float df = nb[e] * sad - na * S[bb[e]][d];
      sq[e] = sq[e] + df * df;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = sq[e] / (na * nb[e] * (na + nb[e]));
}

constexpr int CL_NT = 1024;            // threads of the clustering workgroup
constexpr int CL_SLOTS = CL_NT / SEM_NPK;  // threads per pool key / bucket row

__global__ __launch_bounds__(CL_NT) void sem_cluster_kernel(const unsigned short* __restrict__ kidx,
                                                            long long L_max, SemPaging pg, SemGeom g,
                                                            int first_block, int NB,
                                                            unsigned short* __restrict__ cent,
                                                            int* __restrict__ table, int* __restrict__ offs) {
  __shared__ float S[SEM_NPK][SEM_D + 1];
  __shared__ float C[SEM_NPK][SEM_NPK + 1];
  __shared__ int cnt[SEM_NPK], lab[SEM_NPK], partner[SEM_NPK], into[SEM_NPK], off_of[SEM_NPK];
  __shared__ float pcost[SEM_NPK];
  __shared__ float bcost[CL_SLOTS][SEM_NPK];
  __shared__ int bidx[CL_SLOTS][SEM_NPK];
  __shared__ int pa[SEM_NPK / 2], pb[SEM_NPK / 2], keep[SEM_NPK / 2];
  __shared__ float pc[SEM_NPK / 2];
  __shared__ int id_of_rank[SEM_SLOTS];
  __shared__ int sh_np;

  const int t = threadIdx.x;
  const int blk = first_block + blockIdx.x;
  const int b = blockIdx.y;
  const int npk = g.npk;
  const int row = t & (SEM_NPK - 1), slot = t >> 7;  // a bucket row and one of its CL_SLOTS threads

  // 1. pool keys: the block's keys normalised and summed n_pool at a time, in key order;
  //    each of a pool key's 8 threads divides its 8 dims (the norm needs all 64)
  if (row < npk) {
    float P[8];
    for (int i = 0; i < g.n_pool; ++i) {
      const int j = blk * g.n_cluster + row * g.n_pool + i;
      const uint4* kr = reinterpret_cast<const uint4*>(kidx + pg.row(b, L_max, j) * SEM_D);
      float x[SEM_D];
#pragma unroll
      for (int c = 0; c < 8; ++c) unpack8(kr[c], x + 8 * c);
      float ss = 0.f;
#pragma unroll
      for (int d = 0; d < SEM_D; ++d) ss = ss + x[d] * x[d];
      const float nrm = sqrtf(ss);
      float xs[8];  // this thread's 8 dims, reloaded (a runtime index into x would spill)
      unpack8(kr[slot], xs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = nrm > 0.f ? xs[e] / nrm : 0.f;
        P[e] = i == 0 ? y : P[e] + y;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) S[row][8 * slot + e] = P[e];
  }
  if (t < SEM_NPK) {
    cnt[t] = t < npk ? 1 : 0;
    lab[t] = t;
  }
  __syncthreads();

  // 2. cost of every ordered pair (both triangles; the formula is symmetric bit for bit):
  //    thread (row, slot) takes columns slot, slot + 8, ..., four at a time
  if (row < npk) {
    for (int c0 = slot; c0 < npk; c0 += 4 * CL_SLOTS) {
      int bb[4];
      float nb[4], out[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = c0 + e * CL_SLOTS;
        bb[e] = c < npk ? c : row;
        nb[e] = 1.f;
      }
      ward_cost4(S, row, 1.f, bb, nb, out);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (bb[e] != row) C[row][bb[e]] = out[e];
    }
  }
  __syncthreads();

  // 3. merge rounds
  int live = npk;
  while (live > g.m) {
    // cheapest allowed partner of every bucket: each of its 8 threads scans 16 columns
    // in order, then the lowest (cost, column) of the 8 in slot order
    if (row < npk) {
      int bi = -1;
      float best = 0.f;
      const int ca = cnt[row];
      if (ca > 0) {
        const int c_end = (slot + 1) * (SEM_NPK / CL_SLOTS) < npk ? (slot + 1) * (SEM_NPK / CL_SLOTS) : npk;
        for (int bb = slot * (SEM_NPK / CL_SLOTS); bb < c_end; ++bb) {
          const int cbb = cnt[bb];
          if (bb == row || cbb == 0 || ca + cbb > g.cap) continue;
          const float c = C[row][bb];
          if (bi < 0 || c < best) {
            best = c;
            bi = bb;
          }
        }
      }
      bcost[slot][row] = best;
      bidx[slot][row] = bi;
    }
    if (t == 0) sh_np = 0;
    __syncthreads();
    if (t < npk) {
      int bi = -1;
      float best = 0.f;
      for (int sl = 0; sl < CL_SLOTS; ++sl) {
        const int i2 = bidx[sl][t];
        if (i2 < 0) continue;
        const float c = bcost[sl][t];
        if (bi < 0 || c < best) {
          best = c;
          bi = i2;
        }
      }
      partner[t] = bi;
      pcost[t] = best;
      into[t] = -1;
    }
    __syncthreads();
    if (t < npk) {
      const int bb = partner[t];
      if (bb > t && partner[bb] == t) {
        const int s2 = atomicAdd(&sh_np, 1);
        pa[s2] = t;
        pb[s2] = bb;
        pc[s2] = pcost[t];
      }
    }
    __syncthreads();
    const int np = sh_np;
    if (np == 0) break;
    const int need = live - g.m;
    // all mutual pairs merge, unless that would leave fewer than m buckets: then the
    // cheapest `need` (cost, then lower id)
    if (t < np) {
      int rk = 0;
      if (np > need)
        for (int j = 0; j < np; ++j) rk += (pc[j] < pc[t]) || (pc[j] == pc[t] && pa[j] < pa[t]);
      keep[t] = rk < need;
    }
    __syncthreads();
    for (int x = t; x < np * SEM_D; x += CL_NT) {
      const int s2 = x >> 6, d = x & (SEM_D - 1);
      if (keep[s2]) S[pa[s2]][d] = S[pa[s2]][d] + S[pb[s2]][d];
    }
    if (t < np && keep[t]) {
      into[pb[t]] = pa[t];
      cnt[pa[t]] = cnt[pa[t]] + cnt[pb[t]];
      cnt[pb[t]] = 0;
    }
    __syncthreads();
    if (t < npk) {
      const int l = into[lab[t]];
      if (l >= 0) lab[t] = l;
    }
    live -= np < need ? np : need;
    // costs of every live bucket against the merged ones: thread (row, slot) takes
    // merged pairs slot, slot + 8, ..., four at a time
    if (row < npk && cnt[row] > 0) {
      const float na = (float)cnt[row];
      for (int s0 = slot; s0 < np; s0 += 4 * CL_SLOTS) {
        int bb[4];
        float nb[4], out[4];
        bool use[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s2 = s0 + e * CL_SLOTS;
          use[e] = s2 < np && keep[s2] && pa[s2] != row;
          bb[e] = use[e] ? pa[s2] : row;
          nb[e] = (float)cnt[bb[e]];
        }
        ward_cost4(S, row, na, bb, nb, out);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (use[e]) {
            C[row][bb[e]] = out[e];
            C[bb[e]][row] = out[e];
          }
      }
    }
    __syncthreads();
  }
  // 4. the cache entry: buckets in id order, their keys ascending
  if (t < npk && cnt[t] > 0) {
    int r = 0, o = 0;
    for (int j = 0; j < t; ++j)
      if (cnt[j] > 0) {
        ++r;
        o += cnt[j];
      }
    off_of[t] = o * g.n_pool;
    if (r < SEM_SLOTS) id_of_rank[r] = t;
  }
  __syncthreads();
  const long long cb = pg.slot(b, NB, blk);
  if (t < npk) {
    const int a = lab[t];
    int pos = 0;
    for (int j = 0; j < t; ++j) pos += lab[j] == a;
    int* tb = table + cb * g.n_cluster + off_of[a] + pos * g.n_pool;
    for (int i = 0; i < g.n_pool; ++i) tb[i] = blk * g.n_cluster + t * g.n_pool + i;
  }
  int* ob = offs + cb * (g.m + 1);
  if (t < g.m) ob[t] = off_of[id_of_rank[t]];
  if (t == 0) ob[g.m] = g.n_cluster;
  if (t < SEM_SLOTS) {
    float v[SEM_D];
    if (t < g.m) {
      const int a = id_of_rank[t];
      float ss = 0.f;
#pragma unroll
      for (int d = 0; d < SEM_D; ++d) ss = ss + S[a][d] * S[a][d];
      const float nrm = sqrtf(ss);
#pragma unroll
      for (int d = 0; d < SEM_D; ++d) v[d] = nrm > 0.f ? S[a][d] / nrm : 0.f;
    } else {
#pragma unroll
      for (int d = 0; d < SEM_D; ++d) v[d] = 0.f;
    }
    uint4* cp = reinterpret_cast<uint4*>(cent + cb * (SEM_D * SEM_SLOTS));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 w;
      w.x = to_bf16(v[8 * c + 0]) | (to_bf16(v[8 * c + 1]) << 16);
      w.y = to_bf16(v[8 * c + 2]) | (to_bf16(v[8 * c + 3]) << 16);
      w.z = to_bf16(v[8 * c + 4]) | (to_bf16(v[8 * c + 5]) << 16);
      w.w = to_bf16(v[8 * c + 6]) | (to_bf16(v[8 * c + 7]) << 16);
      cp[c * SEM_SLOTS + t] = w;
    }
  }
}

// ---------------------------------------------------------------------------------
// Index queries: normalised in fp32, rounded to bf16, kept as fp32 values.

__global__ __launch_bounds__(256) void sem_qnorm_kernel(const unsigned short* __restrict__ q, int n_q, int i0, int nqc,
                                                        int rows, float* __restrict__ qn) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int b = r / nqc, i = r - b * nqc;
  const uint4* row = reinterpret_cast<const uint4*>(q + ((long long)b * n_q + i0 + i) * SEM_D);
  float x[SEM_D];
#pragma unroll
  for (int c = 0; c < 8; ++c) unpack8(row[c], x + 8 * c);
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < SEM_D; ++d) ss = ss + x[d] * x[d];
  const float nrm = sqrtf(ss);
  float4* out = reinterpret_cast<float4*>(qn + (long long)r * SEM_D);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = nrm > 0.f ? x[4 * c + e] / nrm : 0.f;
      y[e] = __uint_as_float(to_bf16(v) << 16);
    }
    out[c] = make_float4(y[0], y[1], y[2], y[3]);
  }
}

// ---------------------------------------------------------------------------------
// Scores s_b = c_b . q: one wave per (cluster block, query tile), a lane per bucket
// slot; the lane holds its centroid in registers and takes the tile's queries one by
// one (wave-uniform).  Every score of the blocks before a query's own is written to
// that query's row of the score table; the next block's centroids are loaded while
// the current one is scored.

// ---------------------------------------------------------------------------------
// Selection by threshold, decode rows ("Latent Sparse Attention (LSA)", App. F.1
// "Selection by threshold", "Flat decode").  Before the scan, a threshold theta_i is set
// for each query from a sample of its row; the scan then appends every bucket scoring
// at or above theta_i to the query's list L_i (one comparison per score, whatever the
// span), and the selection ranks only L_i.  When L_i holds every such bucket (it did not
// overflow) and at least p of them, the row's top-p all score >= theta_i and are in it;
// otherwise the row falls back to the scores the scan wrote.  Either way the result is
// the exact top-p: the threshold only sets how many buckets are listed.
constexpr int SEM_LCAP = 4096;     // list entries per row
constexpr int SEM_THR_NT = 1024;   // threads of the threshold workgroup
constexpr int SEM_THR_C = 16;      // sampled buckets per thread (16384 at most)

struct SemList {
  unsigned long long* keys;  // [rows][SEM_LCAP]: order key of the score << 32 | ~bucket
  int* cnt;                  // [rows]: buckets at or above theta (may exceed SEM_LCAP)
  unsigned* theta;           // [rows]: order key of theta
};

// The query normalised as the scan does it (each wave on its own, the same roundings):
// the 64 values wave-uniform.
__device__ __forceinline__ void sem_decode_query(const unsigned short* __restrict__ q_idx, long long qrow, int lane,
                                                 float (&q)[SEM_D]) {
  const float x = __uint_as_float((unsigned)q_idx[qrow * SEM_D + lane] << 16);
  const float sq = x * x;
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < SEM_D; ++d) ss = ss + __shfl(sq, d);
  const float nrm = sqrtf(ss);
  const int yb = (int)(to_bf16(nrm > 0.f ? x / nrm : 0.f) << 16);
#pragma unroll
  for (int d = 0; d < SEM_D; ++d) q[d] = __int_as_float(__builtin_amdgcn_readlane(yb, d));
}

// One workgroup per decode row: theta_i and a cleared list counter.  The sample is
// n_s = N / 8 buckets (2048 to 16384), in runs of 8 neighbouring buckets spread evenly
// over the row, scored exactly as the scan scores them; theta_i is the n_theta-th best
// sampled score with n_theta = 2 p n_s / N, so about 2 p buckets of the row reach it
// (room for the sample's noise on both sides: p below, SEM_LCAP - 2 p above).  Rows of
// at most SEM_LCAP buckets list every bucket.  mode 2 / 3 set theta above / below every
// score, so that every row falls back (tests).
__global__ __launch_bounds__(SEM_THR_NT) void sem_theta_kernel(const unsigned short* __restrict__ q_idx,
                                                               const int* __restrict__ q_pos, int n_q, int i0,
                                                               SemPaging pg, const unsigned short* __restrict__ cent,
                                                               int NB, int m, int n_cluster, int p_top, int mode,
                                                               SemList L) {
  constexpr int NT = SEM_THR_NT, C = SEM_THR_C;
  __shared__ int hist[2048];
  __shared__ int scan_tmp[NT / 64];
  __shared__ int sh[4];
  __shared__ unsigned long long shu[2];
  const int t = threadIdx.x, lane = t & 63, b = blockIdx.x;
  const long long qrow = (long long)b * n_q + i0;
  const int p = q_pos[qrow];
  int nb = p < 0 ? 0 : p / n_cluster;
  nb = nb < NB ? nb : NB;
  const int N = nb * m;
  unsigned theta = 0u;  // every bucket
  if (mode == 2) {
    theta = 0xFFFFFFFFu;
  } else if (mode == 0 && N > SEM_LCAP) {
    float q[SEM_D];
    sem_decode_query(q_idx, qrow, lane, q);
    int n_s = N / 8;
    n_s = n_s < 2048 ? 2048 : (n_s > NT * C ? NT * C : n_s);
    n_s &= ~7;
    const int runs = n_s / 8;
    int n_theta = (int)((2LL * p_top * n_s + N / 2) / N);
    n_theta = n_theta < 1 ? 1 : (n_theta > n_s ? n_s : n_theta);
    const uint4* c4 = reinterpret_cast<const uint4*>(cent);
    unsigned long long key[C];
    unsigned vmask = 0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = c * NT + t;
      key[c] = 0ull;
      if (e < n_s) {
        int j = (int)((long long)(e >> 3) * N / runs) + (e & 7);
        j = j < N ? j : N - 1;
        const int blk = j / m, sl = j - blk * m;
        const uint4* cb = c4 + pg.slot(b, NB, blk) * (SEM_D * SEM_SLOTS / 8) + sl;
        uint4 v[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) v[g] = cb[g * SEM_SLOTS];
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          float cv[8];
          unpack8(v[g], cv);
#pragma unroll
          for (int d = 0; d < 8; ++d) acc = fmaf(q[8 * g + d], cv[d], acc);
        }
        key[c] = ((unsigned long long)order_key(acc) << 32) | (0xFFFFFFFFu - (unsigned)e);
        vmask |= 1u << c;
      }
    }
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, n_theta, hist, scan_tmp, sh, shu, &need_eq);
    theta = (unsigned)(T >> 32);
  }
  if (t == 0) {  // decode rows: one query per sequence, row b
    L.cnt[b] = 0;
    L.theta[b] = theta;
  }
}

// Decode (one query per sequence): the same scores, with the query normalised inside
// each wave -- lane d holds x_d, the sum of squares is taken d = 0, 1, ... across the
// lanes, and the 64 rounded values are then wave-uniform -- so no separate launch.
// With a list (L.keys), every bucket scoring at or above the row's theta is also appended
// to the row's list: one ballot and one counter atomic per wave and block.
__global__ __launch_bounds__(256) void sem_score_decode_kernel(const unsigned short* __restrict__ q_idx,
                                                               const int* __restrict__ q_pos, int n_q, int i0,
                                                               SemPaging pg,
                                                               const unsigned short* __restrict__ cent, int NB,
                                                               int m, int n_cluster, int bpw,
                                                               float* __restrict__ S, long long ld, SemList L) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int blk0 = (blockIdx.x * 4 + w) * bpw;
  if (blk0 >= NB) return;
  const int p = q_pos[(long long)b * n_q + i0];
  const int own = p < 0 ? 0 : p / n_cluster;
  int blk_end = blk0 + (bpw < 4 ? bpw : 4);
  blk_end = blk_end < NB ? blk_end : NB;
  blk_end = blk_end < own ? blk_end : own;
  if (blk0 >= blk_end) return;

  // the wave's (at most 4) blocks: cache entries looked up before any centroid load,
  // the next ones kept in three rotating registers
  const uint4* c4 = reinterpret_cast<const uint4*>(cent);
  const long long s0 = pg.slot(b, NB, blk0);
  long long s1 = blk0 + 1 < blk_end ? pg.slot(b, NB, blk0 + 1) : 0;
  long long s2 = blk0 + 2 < blk_end ? pg.slot(b, NB, blk0 + 2) : 0;
  long long s3 = blk0 + 3 < blk_end ? pg.slot(b, NB, blk0 + 3) : 0;
  uint4 nxt[8];
  {
    const uint4* cb = c4 + s0 * (SEM_D * SEM_SLOTS / 8);
#pragma unroll
    for (int c = 0; c < 8; ++c) nxt[c] = cb[c * SEM_SLOTS + lane];
  }

  float q[SEM_D];  // wave-uniform: scalar registers
  sem_decode_query(q_idx, (long long)b * n_q + i0, lane, q);
  const unsigned theta = L.keys ? L.theta[b] : 0u;

#pragma unroll 1
  for (int blk = blk0; blk < blk_end; ++blk) {
    float cv[SEM_D];
#pragma unroll
    for (int c = 0; c < 8; ++c) unpack8(nxt[c], cv + 8 * c);
    if (blk + 1 < blk_end) {
      const uint4* cb = c4 + s1 * (SEM_D * SEM_SLOTS / 8);
#pragma unroll
      for (int c = 0; c < 8; ++c) nxt[c] = cb[c * SEM_SLOTS + lane];
    }
    s1 = s2;
    s2 = s3;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < SEM_D; ++d) acc = fmaf(q[d], cv[d], acc);
    if (lane < m) S[(long long)b * ld + (long long)blk * m + lane] = acc;
    if (L.keys) {
      const unsigned ok = order_key(acc);
      const bool pass = lane < m && ok >= theta;
      const unsigned long long ball = __ballot(pass);
      if (ball != 0ull) {
        int slot0 = 0;
        if (lane == 0) slot0 = atomicAdd(&L.cnt[b], __popcll(ball));
        slot0 = __shfl(slot0, 0);
        const int sl = slot0 + lanes_below(ball);
        if (pass && sl < SEM_LCAP)
          L.keys[(long long)b * SEM_LCAP + sl] =
              ((unsigned long long)ok << 32) | (0xFFFFFFFFu - (unsigned)(blk * m + lane));
      }
    }
  }
}

template <int QT>
__global__ __launch_bounds__(256) void sem_score_kernel(const float* __restrict__ qn, const int* __restrict__ q_pos,
                                                        int n_q, int i0, int nqc, SemPaging pg,
                                                        const unsigned short* __restrict__ cent, int NB, int m,
                                                        int n_cluster, int bpw, float* __restrict__ S, long long ld) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int q0 = blockIdx.y * QT;
  const int blk0 = (blockIdx.x * 4 + w) * bpw;
  if (blk0 >= NB) return;
  // the tile's furthest own block bounds the blocks worth loading
  int own_max = 0;
  for (int qi = 0; qi < QT && q0 + qi < nqc; ++qi) {
    const int p = q_pos[(long long)b * n_q + i0 + q0 + qi];
    const int o = p < 0 ? 0 : p / n_cluster;
    own_max = o > own_max ? o : own_max;
  }
  int blk_end = blk0 + (bpw < 4 ? bpw : 4);
  blk_end = blk_end < NB ? blk_end : NB;
  blk_end = blk_end < own_max ? blk_end : own_max;
  if (blk0 >= blk_end) return;

  // the wave's (at most 4) blocks: cache entries looked up before any centroid load,
  // the next ones kept in three rotating registers
  const uint4* c4 = reinterpret_cast<const uint4*>(cent);
  const long long s0 = pg.slot(b, NB, blk0);
  long long s1 = blk0 + 1 < blk_end ? pg.slot(b, NB, blk0 + 1) : 0;
  long long s2 = blk0 + 2 < blk_end ? pg.slot(b, NB, blk0 + 2) : 0;
  long long s3 = blk0 + 3 < blk_end ? pg.slot(b, NB, blk0 + 3) : 0;
  uint4 nxt[8];
  {
    const uint4* cb = c4 + s0 * (SEM_D * SEM_SLOTS / 8);
#pragma unroll
    for (int c = 0; c < 8; ++c) nxt[c] = cb[c * SEM_SLOTS + lane];
  }
#pragma unroll 1
  for (int blk = blk0; blk < blk_end; ++blk) {
    float cv[SEM_D];
#pragma unroll
    for (int c = 0; c < 8; ++c) unpack8(nxt[c], cv + 8 * c);
    if (blk + 1 < blk_end) {
      const uint4* cb = c4 + s1 * (SEM_D * SEM_SLOTS / 8);
#pragma unroll
      for (int c = 0; c < 8; ++c) nxt[c] = cb[c * SEM_SLOTS + lane];
    }
    s1 = s2;
    s2 = s3;
    for (int qi = 0; qi < QT; ++qi) {
      const int i = q0 + qi;
      if (i >= nqc) break;
      const int p = q_pos[(long long)b * n_q + i0 + i];
      if (p < 0 || blk >= p / n_cluster) continue;
      const float* q = qn + ((long long)b * nqc + i) * SEM_D;
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < SEM_D; ++d) acc = fmaf(q[d], cv[d], acc);
      if (lane < m) S[((long long)b * nqc + i) * ld + (long long)blk * m + lane] = acc;
    }
  }
}

// ---------------------------------------------------------------------------------
// Selection and expansion: one workgroup per query.  The top-p buckets by packed key
// (order key of the score above, inverted bucket id below) come from a radix select
// over the score row (four 8-bit digits) and one ordered pass that takes every bucket
// above the cut and the lowest-id ones at it.  They are sorted best first, their keys
// outside the sink and the window counted, and the long-range keys written up to k
// (the bucket at the cut in part); the list is sink, long-range keys ascending, window.

constexpr int SEM_PMAX = 2048;
constexpr int SEM_KMAX = 4096;
constexpr int SEM_LPT = 4096;  // page-table entries of one sequence staged in LDS (256K keys of 64-key pages)
constexpr int SEM_KC = 8192;   // candidates of a long row's chunks (chunks * p_top at most)

__global__ __launch_bounds__(SEL_NT) void sem_select_stream_kernel(const float* __restrict__ S, long long ld,
                                                            const int* __restrict__ q_pos, int n_q, int i0, int nqc,
                                                            SemPaging pg,
                                                            const int* __restrict__ table, const int* __restrict__ offs,
                                                            int NB, int m, int n_cluster, int k, int p_top, int n_sink,
                                                            int n_w, int W, int* __restrict__ idx,
                                                            int* __restrict__ count) {
  __shared__ unsigned long long K[SEM_PMAX];
  __shared__ int avail[SEM_PMAX];
  __shared__ int excl[SEM_PMAX];
  __shared__ int LR[SEM_KMAX];
  __shared__ int hist[256];
  __shared__ int scan_tmp[SEL_NT / 64];
  __shared__ int sh[4];

  const int t = threadIdx.x;
  const int i = blockIdx.x, b = blockIdx.y;
  const long long qrow = (long long)b * n_q + i0 + i;
  const int p = q_pos[qrow];
  int* out = idx + qrow * W;
  if (p < 0) {
    for (int j = t; j < W; j += SEL_NT) out[j] = -1;
    if (t == 0) count[qrow] = 0;
    return;
  }
  int nb = p / n_cluster;
  nb = nb < NB ? nb : NB;
  const int N = nb * m;
  const float* row = S + ((long long)b * nqc + i) * ld;
  const int w0 = p - n_w + 1 > 0 ? p - n_w + 1 : 0;

  int nk;
  if (N <= p_top) {
    for (int j = t; j < N; j += SEL_NT)
      K[j] = ((unsigned long long)order_key(row[j]) << 32) | (0xFFFFFFFFu - (unsigned)j);
    nk = N;
  } else {
    unsigned prefix = 0;
    int need = p_top;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int j = t; j < 256; j += SEL_NT) hist[j] = 0;
      __syncthreads();
      const unsigned hi_mask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int j = t; j < N; j += SEL_NT) {
        const unsigned u = order_key(row[j]);
        if ((u & hi_mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (t == 0) {
        int acc = 0, dg = 255;
        for (; dg > 0; --dg) {
          if (acc + hist[dg] >= need) break;
          acc += hist[dg];
        }
        sh[0] = dg;
        sh[1] = need - acc;
      }
      __syncthreads();
      prefix |= (unsigned)sh[0] << shift;
      need = sh[1];
      __syncthreads();
    }
    // every key above `prefix`, and the `need` lowest-id keys equal to it
    if (t == 0) {
      sh[2] = 0;
      sh[3] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += SEL_NT) {
      const int j = base + t;
      unsigned u = 0;
      if (j < N) u = order_key(row[j]);
      const bool gt = j < N && u > prefix, eq = j < N && u == prefix;
      int eq_total;
      const int eq_rank = block_exclusive_scan<SEL_NT>(eq ? 1 : 0, scan_tmp, &eq_total);
      const int eq_base = sh[3];
      if (gt || (eq && eq_base + eq_rank < need)) {
        const int s = atomicAdd(&sh[2], 1);
        K[s] = ((unsigned long long)u << 32) | (0xFFFFFFFFu - (unsigned)j);
      }
      __syncthreads();
      if (t == 0) sh[3] = eq_base + eq_total;
      __syncthreads();
    }
    nk = p_top;
  }

  // best first: bitonic sort of the packed keys, descending (padding 0 sorts last)
  int P2 = 1;
  while (P2 < nk) P2 <<= 1;
  for (int j = nk + t; j < P2; j += SEL_NT) K[j] = 0;
  __syncthreads();
  for (int kk = 2; kk <= P2; kk <<= 1)
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int x = t; x < P2; x += SEL_NT) {
        const int y = x ^ jj;
        if (y > x) {
          const unsigned long long a0 = K[x], a1 = K[y];
          const bool desc = (x & kk) == 0;
          if (desc ? (a0 < a1) : (a0 > a1)) {
            K[x] = a1;
            K[y] = a0;
          }
        }
      }
      __syncthreads();
    }

  // keys each selected bucket offers outside the sink and the window
  for (int r = t; r < nk; r += SEL_NT) {
    const int gid = (int)(0xFFFFFFFFu - (unsigned)(K[r] & 0xFFFFFFFFull));
    const int blk = gid / m, loc = gid - blk * m;
    const long long sl = pg.slot(b, NB, blk);
    const int* ob = offs + sl * (m + 1);
    const int o0 = ob[loc], o1 = ob[loc + 1];
    int av = o1 - o0;
    if (blk * n_cluster < n_sink || (blk + 1) * n_cluster > w0) {
      const int* tb = table + sl * n_cluster;
      av = 0;
      for (int x = o0; x < o1; ++x) {
        const int key = tb[x];
        av += key >= n_sink && key < w0;
      }
    }
    avail[r] = av;
  }
  __syncthreads();
  // exclusive scan over the best-first order: each thread a contiguous run
  const int per = (nk + SEL_NT - 1) / SEL_NT;
  int run = 0;
  for (int e = 0; e < per; ++e) {
    const int r = t * per + e;
    if (r < nk) run += avail[r];
  }
  int total;
  int pre = block_exclusive_scan<SEL_NT>(run, scan_tmp, &total);
  for (int e = 0; e < per; ++e) {
    const int r = t * per + e;
    if (r < nk) {
      excl[r] = pre;
      pre += avail[r];
    }
  }
  __syncthreads();
  const int n_lr = total < k ? total : k;
  for (int r = t; r < nk; r += SEL_NT) {
    const int e0 = excl[r];
    if (e0 >= k) continue;
    const int take = avail[r] < k - e0 ? avail[r] : k - e0;
    const int gid = (int)(0xFFFFFFFFu - (unsigned)(K[r] & 0xFFFFFFFFull));
    const int blk = gid / m, loc = gid - blk * m;
    const long long sl = pg.slot(b, NB, blk);
    const int* ob = offs + sl * (m + 1);
    const int* tb = table + sl * n_cluster;
    int n = 0;
    for (int x = ob[loc]; x < ob[loc + 1] && n < take; ++x) {
      const int key = tb[x];
      if (key >= n_sink && key < w0) LR[e0 + n++] = key;
    }
  }
  // long-range keys ascending
  int Q2 = 1;
  while (Q2 < n_lr) Q2 <<= 1;
  for (int j = n_lr + t; j < Q2; j += SEL_NT) LR[j] = 0x7FFFFFFF;
  __syncthreads();
  for (int kk = 2; kk <= Q2; kk <<= 1)
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int x = t; x < Q2; x += SEL_NT) {
        const int y = x ^ jj;
        if (y > x) {
          const int a0 = LR[x], a1 = LR[y];
          const bool asc = (x & kk) == 0;
          if (asc ? (a0 > a1) : (a0 < a1)) {
            LR[x] = a1;
            LR[y] = a0;
          }
        }
      }
      __syncthreads();
    }
  const int n_s = n_sink < w0 ? n_sink : w0;
  const int n_win = p - w0 + 1;
  const int cnt_all = n_s + n_lr + n_win;
  for (int j = t; j < W; j += SEL_NT) {
    int v = -1;
    if (j < n_s) v = j;
    else if (j < n_s + n_lr) v = LR[j - n_s];
    else if (j < cnt_all) v = w0 + (j - n_s - n_lr);
    out[j] = v < 0 ? v : pg.list_entry(b, v);
  }
  if (t == 0) count[qrow] = cnt_all;
}


// Long rows with few queries: one workgroup per (span of SPAN_B buckets, query) keeps the
// span's top-p (registers, radix cut, ties to the lowest id) and writes them as packed
// keys over the start of its own span of the score row, after a count: [count][keys...]
// (the span is read whole before anything is written; spans are disjoint).
constexpr int SPAN_B = 1024 * 16;
__global__ __launch_bounds__(1024) void sem_span_topk_kernel(float* __restrict__ S, long long ld,
                                                             const int* __restrict__ q_pos, int n_q, int i0, int nqc,
                                                             int NB, int m, int n_cluster, int p_top) {
  constexpr int NT = 1024, C = 16, NWD = NT * C / 32;
  __shared__ int hist[2048];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ int scan_tmp[NT / 64];
  __shared__ int sh[4];
  __shared__ unsigned long long shu[2];
  const int t = threadIdx.x, span = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const int p = q_pos[(long long)b * n_q + i0 + i];
  if (p < 0) return;
  int nb = p / n_cluster;
  nb = nb < NB ? nb : NB;
  const int N = nb * m, base = span * SPAN_B;
  if (base >= N) return;
  float* row = S + ((long long)b * nqc + i) * ld;
  unsigned long long key[C];
  unsigned vmask = 0u;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = base + c * NT + t;
    key[c] = 0ull;
    if (j < N) {
      key[c] = order_key(row[j]);
      vmask |= 1u << c;
    }
  }
  const int Nc = N - base < SPAN_B ? N - base : SPAN_B;
  if (Nc > p_top) {
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, p_top, hist, scan_tmp, sh, shu, &need_eq);
    mark_kept64<NT, C>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
  }
  if (t == 0) sh[2] = 0;
  __syncthreads();  // every score of the span is in registers before the span is overwritten
  unsigned long long* out = reinterpret_cast<unsigned long long*>(row + base);
  const int lane = t & 63;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int pos = c * NT + t;
    const bool kept = ((vmask >> c) & 1u) && (Nc <= p_top || ((bm[pos >> 5] >> (pos & 31)) & 1u));
    const unsigned long long ball = __ballot(kept);
    if (ball == 0ull) continue;
    int slot0 = 0;
    if (lane == 0) slot0 = atomicAdd(&sh[2], __popcll(ball));
    slot0 = __shfl(slot0, 0);
    if (kept) out[1 + slot0 + lanes_below(ball)] = (key[c] << 32) | (0xFFFFFFFFu - (unsigned)(base + pos));
  }
  __syncthreads();
  if (t == 0) out[0] = (unsigned long long)sh[2];
}

// Selection and expansion of rows of at most NT * C buckets whose long-range keys lie
// below 32 * SelLbm<C>::WORDS positions: one NT-thread workgroup per query, the row's
// order keys in registers (bucket c * NT + t in slot c of thread t).  The cut is a
// radix select over them (11-bit digits below the bits all keys share; ties to the
// lowest bucket id); the kept buckets' packed keys, appended from the registers, are
// sorted best first (lane shuffles for exchanges under 64 apart, LDS above); each
// bucket's offsets, eligible-key mask and long-range keys are handled by the thread
// owning its run of that order, one scan giving every bucket's start; the long-range
// keys are marked in an LDS bitmap of key positions, which yields them ascending.
// MINW > 1 holds the kernel to the registers of MINW waves per SIMD (two workgroups
// per compute unit when many rows run).
template <int C>
struct SelLbm {
  static constexpr int WORDS = 256 * C;  // positions < 8192 * C: n_bavg = 8 fills it
};

template <int NT, int C, int MINW, bool PAGED, bool LONG>
__global__ __launch_bounds__(NT, MINW) void sem_select_kernel(const float* __restrict__ S, long long ld,
                                                             const int* __restrict__ q_pos, int n_q, int i0, int nqc,
                                                             const int* __restrict__ table,
                                                             const int* __restrict__ offs, int NB, int m,
                                                             int n_cluster, int n_bmax, int k, int p_top, int n_sink,
                                                             int n_w, int W, int* __restrict__ idx,
                                                             int* __restrict__ count, SemPaging pg, int split,
                                                             SemList lst) {
  constexpr int NWD = NT * C / 32;
  constexpr int LW = SelLbm<C>::WORDS;
  __shared__ unsigned long long K[SEM_PMAX];
  __shared__ int hist[2048];
  __shared__ unsigned bm[NWD], eqm[NWD];
  __shared__ unsigned lbm[LONG ? 1 : LW];
  __shared__ unsigned long long Kc[LONG ? SEM_KC : 1];  // chunks' candidates (long rows)
  __shared__ int LRs[LONG ? SEM_KMAX : 1];               // long-range keys to sort (long rows)
  __shared__ int scan_tmp[NT / 64];
  __shared__ int sh[4];
  __shared__ unsigned long long shu[2];
  __shared__ int lpt[PAGED ? SEM_LPT : 1];  // the sequence's page-table row (clamped), when it fits

  const int t = threadIdx.x;
  const int i = blockIdx.x, b = blockIdx.y;
  const long long qrow = (long long)b * n_q + i0 + i;
  const int p = q_pos[qrow];
  int* out = idx + qrow * W;
  if (p < 0) {
    for (int j = t; j < W; j += NT) out[j] = -1;
    if (t == 0) count[qrow] = 0;
    return;
  }
  int nb = p / n_cluster;
  nb = nb < NB ? nb : NB;
  const int N = nb * m;
  const float* row = S + ((long long)b * nqc + i) * ld;
  const int w0 = p - n_w + 1 > 0 ? p - n_w + 1 : 0;
  const bool lds_pt = PAGED && pg.pt && pg.max_pages <= SEM_LPT;
  const int pmask = (1 << pg.plog2) - 1;
  auto entry = [&](int j) -> int {
    if (!PAGED) return j;
    if (!lds_pt) return pg.list_entry(b, j);
    int pi = j >> pg.plog2;
    pi = pi < pg.max_pages ? pi : pg.max_pages - 1;
    return (lpt[pi] << pg.plog2) | (j & pmask);
  };

  // 1. the kept buckets, marked in bm by bucket id
  int nk;
  if constexpr (LONG) {
    // rows longer than the registers hold: every chunk of NT * C buckets keeps its own
    // top-p (the row's top-p is among them), as packed keys with the global bucket id
    if (lds_pt)
      for (int x = t; x < pg.max_pages; x += NT) {
        long long v = pg.pt[(long long)b * pg.max_pages + x];
        lpt[x] = (int)(v < 0 ? 0 : (v >= pg.n_pages ? pg.n_pages - 1 : v));
      }
    constexpr int CH = NT * C;
    if (t == 0) sh[3] = 0;
    __syncthreads();  // a row with no scored bucket reads sh[3] with no other barrier
    const int lane = t & 63;
    // the row's threshold list, when it holds every bucket at or above theta and at least
    // p_top of them (then the row's top-p is in it); otherwise the whole row below
    bool listed = false;
    if (lst.keys) {
      const long long lr = (long long)b * nqc + i;
      const int c = lst.cnt[lr];
      if (c >= p_top && c <= SEM_LCAP) {
        for (int x = t; x < c; x += NT) Kc[x] = lst.keys[lr * SEM_LCAP + x];
        __syncthreads();
        if (t == 0) sh[3] = c;
        __syncthreads();
        listed = true;
      }
    }
    if (split && !listed) {
      // the spans' candidates, left in the score row by sem_span_topk_kernel (every
      // thread reads every count, so all keep the same running offset)
      int off = 0;
      for (int base = 0; base < N; base += SPAN_B) {
        const unsigned long long* cin = reinterpret_cast<const unsigned long long*>(row + base);
        const int cnt_s = (int)cin[0];
        for (int x = t; x < cnt_s; x += NT) Kc[off + x] = cin[1 + x];
        off += cnt_s;
      }
      __syncthreads();
      if (t == 0) sh[3] = off;
      __syncthreads();
    }
    for (int base = 0; base < (split || listed ? 0 : N); base += CH) {
      unsigned long long key[C];
      unsigned vmask = 0u;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int j = base + c * NT + t;
        key[c] = 0ull;
        if (j < N) {
          key[c] = order_key(row[j]);
          vmask |= 1u << c;
        }
      }
      const int Nc = N - base < CH ? N - base : CH;
      if (Nc > p_top) {
        int need_eq;
        const unsigned long long T = radix_cut64<NT, C>(key, vmask, p_top, hist, scan_tmp, sh, shu, &need_eq);
        mark_kept64<NT, C>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int pos = c * NT + t;
        const bool kept = ((vmask >> c) & 1u) && (Nc <= p_top || ((bm[pos >> 5] >> (pos & 31)) & 1u));
        const unsigned long long ball = __ballot(kept);
        if (ball == 0ull) continue;
        int slot0 = 0;
        if (lane == 0) slot0 = atomicAdd(&sh[3], __popcll(ball));
        slot0 = __shfl(slot0, 0);
        if (kept) Kc[slot0 + lanes_below(ball)] = (key[c] << 32) | (0xFFFFFFFFu - (unsigned)(base + pos));
      }
      __syncthreads();
    }
    // the row's top-p among the candidates (packed keys are distinct: no ties)
    const int ncand = sh[3];
    if (ncand > p_top) {
      constexpr int C2 = SEM_KC / NT;
      unsigned long long k2[C2];
      unsigned vm2 = 0u;
#pragma unroll
      for (int c = 0; c < C2; ++c) {
        const int x = c * NT + t;
        k2[c] = x < ncand ? Kc[x] : 0ull;
        if (x < ncand) vm2 |= 1u << c;
      }
      int need_eq;
      const unsigned long long T2 = radix_cut64<NT, C2>(k2, vm2, p_top, hist, scan_tmp, sh, shu, &need_eq);
      mark_kept64<NT, C2>(k2, vm2, T2, need_eq, bm, eqm, scan_tmp);
      if (t == 0) sh[2] = 0;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < C2; ++c) {
        const int pos = c * NT + t;
        const bool kept = ((vm2 >> c) & 1u) && ((bm[pos >> 5] >> (pos & 31)) & 1u);
        const unsigned long long ball = __ballot(kept);
        if (ball == 0ull) continue;
        int slot0 = 0;
        if (lane == 0) slot0 = atomicAdd(&sh[2], __popcll(ball));
        slot0 = __shfl(slot0, 0);
        if (kept) K[slot0 + lanes_below(ball)] = k2[c];
      }
      __syncthreads();
      nk = sh[2];
    } else {
      for (int x = t; x < ncand; x += NT) K[x] = Kc[x];
      __syncthreads();
      nk = ncand;
    }
  } else {
  unsigned long long key[C];
  unsigned vmask = 0u;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = c * NT + t;
    key[c] = 0ull;
    if (j < N) {
      key[c] = order_key(row[j]);
      vmask |= 1u << c;
    }
  }
  // the page-table row, staged for the list's pool rows at the end (read after the
  // barriers of the steps below)
  if (lds_pt)
    for (int x = t; x < pg.max_pages; x += NT) {
      long long v = pg.pt[(long long)b * pg.max_pages + x];
      lpt[x] = (int)(v < 0 ? 0 : (v >= pg.n_pages ? pg.n_pages - 1 : v));
    }
  if (N > p_top) {
    int need_eq;
    const unsigned long long T = radix_cut64<NT, C>(key, vmask, p_top, hist, scan_tmp, sh, shu, &need_eq);
    mark_kept64<NT, C>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
  }
  // the kept buckets' packed keys, appended from the registers (wave-aggregated slots;
  // their order is set by the sort below)
  if (t == 0) sh[2] = 0;
  __syncthreads();
  const int lane = t & 63;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int pos = c * NT + t;
    const bool kept = ((vmask >> c) & 1u) && (N <= p_top || ((bm[pos >> 5] >> (pos & 31)) & 1u));
    const unsigned long long ball = __ballot(kept);
    if (ball == 0ull) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&sh[2], __popcll(ball));
    base = __shfl(base, 0);
    if (kept) K[base + lanes_below(ball)] = (key[c] << 32) | (0xFFFFFFFFu - (unsigned)pos);
  }
  __syncthreads();
  nk = sh[2];
  }

  // 2. best first: bitonic sort of the packed keys, descending (padding 0 sorts last);
  //    one key per thread, exchanges under 64 apart by lane shuffles, wider ones
  //    through LDS
  int P2 = 1;
  while (P2 < nk) P2 <<= 1;
  if (P2 <= NT) {
    unsigned long long v = t < nk ? K[t] : 0ull;
    for (int kk = 2; kk <= P2; kk <<= 1)
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        unsigned long long pv;
        if (jj >= 64) {
          __syncthreads();
          K[t] = v;
          __syncthreads();
          pv = K[t ^ jj];
        } else {
          pv = __shfl_xor(v, jj);
        }
        const bool desc = (t & kk) == 0, lower = (t & jj) == 0;
        v = (desc == lower) ? (v > pv ? v : pv) : (v < pv ? v : pv);
      }
    __syncthreads();
    if (t < P2) K[t] = v;
  } else {
    for (int j = nk + t; j < P2; j += NT) K[j] = 0;
    __syncthreads();
    for (int kk = 2; kk <= P2; kk <<= 1)
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int x = t; x < P2; x += NT) {
          const int y = x ^ jj;
          if (y > x) {
            const unsigned long long a0 = K[x], a1 = K[y];
            const bool desc = (x & kk) == 0;
            if (desc ? (a0 < a1) : (a0 > a1)) {
              K[x] = a1;
              K[y] = a0;
            }
          }
        }
        __syncthreads();
      }
  }
  __syncthreads();

  // 3. each kept bucket, by the thread owning its run of the best-first order: where
  //    its keys start and how many (one load), which of them lie outside the sink and
  //    the window (loads 8 at a time, a 64-bit mask kept in a register), and the
  //    running count of those in best-first order (one scan)
  // long-range keys lie below both the window and the end of the scored blocks
  const int pos_lim = w0 < nb * n_cluster ? w0 : nb * n_cluster;
  const int nlw = (pos_lim + 31) >> 5;
  if constexpr (!LONG)
    for (int wd = t; wd < nlw; wd += NT) lbm[wd] = 0u;
  constexpr int OWN = SEM_PMAX / NT;  // buckets a thread owns, at most
  const int per = (nk + NT - 1) / NT;
  long long o_start[OWN];
  int o_size[OWN];
  unsigned long long o_mask[OWN];
  int run = 0;
#pragma unroll
  for (int e = 0; e < OWN; ++e) {
    const int r = t * per + e;
    o_start[e] = 0;
    o_size[e] = 0;
    o_mask[e] = 0ull;
    if (e >= per || r >= nk) continue;
    const int gid = (int)(0xFFFFFFFFu - (unsigned)(K[r] & 0xFFFFFFFFull));
    const int blk = gid / m, loc = gid - blk * m;
    const long long sl = PAGED ? pg.slot(b, NB, blk) : (long long)b * NB + blk;
    const int* ob = offs + sl * (m + 1);
    const int o0 = ob[loc], o1 = ob[loc + 1];
    o_start[e] = sl * n_cluster + o0;
    o_size[e] = o1 - o0;
    const int* tb = table + o_start[e];
    unsigned long long msk = 0ull;
    for (int base = 0; base < o_size[e]; base += 8) {
      int v[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) v[x] = base + x < o_size[e] ? tb[base + x] : -1;
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if (v[x] >= n_sink && v[x] < w0) msk |= 1ull << (base + x);
    }
    o_mask[e] = msk;
    run += __popcll(msk);
  }
  int total;
  const int pre = block_exclusive_scan<NT>(run, scan_tmp, &total);

  // 4. long-range keys: whole buckets before the cut, the first keys of the one at it
  //    (a key's rank among its bucket's eligible keys is the mask's count below it)
  const int n_lr = total < k ? total : k;
  int e0 = pre;
#pragma unroll
  for (int e = 0; e < OWN; ++e) {
    const unsigned long long msk = o_mask[e];
    const int av = __popcll(msk);
    if (e0 < k && msk != 0ull) {
      const int take = av < k - e0 ? av : k - e0;
      const int* tb = table + o_start[e];
      for (int base = 0; base < o_size[e]; base += 8) {
        int v[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) v[x] = base + x < o_size[e] ? tb[base + x] : -1;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int sl = base + x;
          if (sl < o_size[e] && ((msk >> sl) & 1ull)) {
            const int rank = __popcll(msk & ((1ull << sl) - 1ull));
            if (rank < take) {
              if constexpr (LONG)
                LRs[e0 + rank] = v[x];
              else
                atomicOr(&lbm[v[x] >> 5], 1u << (v[x] & 31));
            }
          }
        }
      }
    }
    e0 += av;
  }
  __syncthreads();
  const int n_s = n_sink < w0 ? n_sink : w0;
  if constexpr (LONG) {
    // the long-range keys ascending: bitonic sort (padding sorts last); up to 2 * NT keys
    // two per thread (keys t and t + NT), exchanges within a thread or under 64 apart
    // without LDS, wider ones through it
    int Q2 = 1;
    while (Q2 < n_lr) Q2 <<= 1;
    if (Q2 <= 2 * NT && Q2 >= 128) {
      int v0 = t < n_lr ? LRs[t] : 0x7FFFFFFF;
      int v1 = t + NT < n_lr ? LRs[t + NT] : 0x7FFFFFFF;
      const bool two = Q2 > NT;
      for (int kk = 2; kk <= Q2; kk <<= 1)
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
          if (jj == NT) {
            // partners are the two keys of this thread: element t (lower) and t + NT
            const bool asc = (t & kk) == 0;
            const int lo = v0 < v1 ? v0 : v1, hi = v0 < v1 ? v1 : v0;
            v0 = asc ? lo : hi;
            v1 = asc ? hi : lo;
            continue;
          }
          int p0, p1;
          if (jj >= 64) {
            __syncthreads();
            LRs[t] = v0;
            if (two) LRs[t + NT] = v1;
            __syncthreads();
            p0 = LRs[t ^ jj];
            p1 = two ? LRs[(t + NT) ^ jj] : 0;
          } else {
            p0 = __shfl_xor(v0, jj);
            p1 = __shfl_xor(v1, jj);
          }
          const int x0 = t, x1 = t + NT;
          const bool asc0 = (x0 & kk) == 0, low0 = (x0 & jj) == 0;
          const bool asc1 = (x1 & kk) == 0, low1 = (x1 & jj) == 0;
          v0 = (asc0 == low0) ? (v0 < p0 ? v0 : p0) : (v0 > p0 ? v0 : p0);
          if (two) v1 = (asc1 == low1) ? (v1 < p1 ? v1 : p1) : (v1 > p1 ? v1 : p1);
        }
      __syncthreads();
      if (t < Q2) LRs[t] = v0;
      if (two && t + NT < Q2) LRs[t + NT] = v1;
      __syncthreads();
    } else {
    for (int x = n_lr + t; x < Q2; x += NT) LRs[x] = 0x7FFFFFFF;
    __syncthreads();
    for (int kk = 2; kk <= Q2; kk <<= 1)
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int x = t; x < Q2; x += NT) {
          const int y = x ^ jj;
          if (y > x) {
            const int a0 = LRs[x], a1 = LRs[y];
            const bool asc = (x & kk) == 0;
            if (asc ? (a0 > a1) : (a0 < a1)) {
              LRs[x] = a1;
              LRs[y] = a0;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int r = t; r < n_lr; r += NT) out[n_s + r] = entry(LRs[r]);
  } else {
    emit_marked<NT>(lbm, nlw, scan_tmp, [&](int r, int pos) { out[n_s + r] = entry(pos); });
  }
  const int n_win = p - w0 + 1;
  const int cnt_all = n_s + n_lr + n_win;
  for (int j = t; j < W; j += NT) {
    if (j < n_s) out[j] = entry(j);
    else if (j >= n_s + n_lr) out[j] = j < cnt_all ? entry(w0 + (j - n_s - n_lr)) : -1;
  }
  if (t == 0) count[qrow] = cnt_all;
}

}  // namespace

// ---------------------------------------------------------------------------------

static SemPaging paging_of(const SemPages& p) {
  SemPaging g;
  g.bt = p.block_table;
  g.n_bslots = p.n_bslots;
  g.pt = p.page_table;
  g.plog2 = 0;
  while (p.page_size > 0 && (1 << g.plog2) < p.page_size) ++g.plog2;
  g.max_pages = p.max_pages;
  g.n_pages = p.page_size > 0 ? p.n_slots / p.page_size : 0;
  return g;
}

hipError_t launch_sem_cluster(const void* k_idx, int B, int L_max, const SemParams& sp, int NB, int first_block,
                              int n_update, void* cent, int32_t* table, int32_t* offs, const SemPages& pages,
                              hipStream_t st) {
  SemGeom g;
  g.n_cluster = sp.n_cluster;
  g.n_pool = sp.n_pool;
  g.npk = sp.n_cluster / sp.n_pool;
  g.m = sp.n_cluster / sp.n_bavg;
  g.cap = sp.n_bmax / sp.n_pool;
  dim3 grid(n_update, B);
  hipLaunchKernelGGL(sem_cluster_kernel, grid, dim3(CL_NT), 0, st, static_cast<const unsigned short*>(k_idx),
                     (long long)L_max, paging_of(pages), g, first_block, NB, static_cast<unsigned short*>(cent), table,
                     offs);
  return hipGetLastError();
}

// Whether a selection kernel with rows of nt * C buckets in registers (C per thread)
// takes rows of n_max buckets whose long-range keys lie below pos_max: the bucket
// count, the position bitmap (32 * SelLbm<C>::WORDS positions) and the bucket size.
static bool sem_fits_registers(long long n_max, long long pos_max, int n_bmax, int nt, int C) {
  return n_max <= (long long)nt * C && pos_max <= 32LL * 256 * C && n_bmax <= 64;
}

// Rows that no register instance takes go through the long-row path, whose span kernel
// writes each span's candidates over the start of its own span of the score row.
static bool sem_long_rows(int NB, int m, int n_cluster, int n_bmax) {
  return !sem_fits_registers((long long)NB * m, (long long)NB * n_cluster, n_bmax, 1024, 32);
}

// Score-row stride: a row's buckets, and for rows of the long-row path room for the last
// span's candidates, which take 2 * (kept + 1) floats where a short last span may hold
// fewer scores than that.
long long sem_ld(int NB, int m, int n_cluster, int n_bmax) {
  long long n = (long long)NB * m;
  if (sem_long_rows(NB, m, n_cluster, n_bmax)) n += 2 * (SEM_MAX_P + 1);
  return (n + 3) / 4 * 4;
}

// Rows that may take the threshold list: decode rows longer than the list.  Each gets
// the list, its count and its threshold after the score rows.
static bool sem_list_rows(int NB, int m, bool decode) { return decode && (long long)NB * m > SEM_LCAP; }

size_t sem_select_row_bytes(int NB, int m, int n_cluster, int n_bmax, bool decode) {
  const size_t lst = sem_list_rows(NB, m, decode) ? (size_t)SEM_LCAP * 8 + 8 : 0;
  return (size_t)SEM_D * 4 + (size_t)sem_ld(NB, m, n_cluster, n_bmax) * 4 + lst;
}

hipError_t launch_sem_select(const SemSelectArgs& a, hipStream_t st) {
  const int m = a.sp.n_cluster / a.sp.n_bavg;
  const long long ld = sem_ld(a.NB, m, a.sp.n_cluster, a.sp.n_bmax);
  const bool decode = a.n_q == 1;
  const size_t row_bytes = sem_select_row_bytes(a.NB, m, a.sp.n_cluster, a.sp.n_bmax, decode);
  const long long rows_fit = (long long)(a.ws_bytes / row_bytes);
  long long nqc_max = rows_fit / a.B;
  if (nqc_max > a.n_q) nqc_max = a.n_q;
  if (nqc_max < 1) return hipErrorInvalidValue;
  const int W = a.n_sink + a.k + a.n_w;
  const SemPaging pg = paging_of(a.pages);
  for (int i0 = 0; i0 < a.n_q; i0 += (int)nqc_max) {
    const int nqc = (int)(a.n_q - i0 < nqc_max ? a.n_q - i0 : nqc_max);
    const int rows = a.B * nqc;
    float* qn = static_cast<float*>(a.ws);
    float* S = qn + (size_t)rows * SEM_D;
    // the threshold list (decode rows longer than the list; the long-row selection ranks
    // it), when asked for: p_top <= SEM_LCAP / 4 (2 p_top expected in the list, room for
    // the noise on both sides), rows the long-row selection takes.  Not the default: the
    // selection's time is the ordering and expansion of the kept buckets, whatever it
    // ranks, so the threshold's extra launch costs more than ranking the whole row here.
    const long long n_max = (long long)a.NB * m, pos_max = (long long)a.NB * a.sp.n_cluster;
    const bool use_list = sem_list_rows(a.NB, m, decode) && a.sp.select_mode != 0 && 4 * a.p_top <= SEM_LCAP &&
                          a.sp.n_bmax <= 64 && (n_max + SPAN_B - 1) / SPAN_B * a.p_top <= SEM_KC;
    SemList L{};
    if (sem_list_rows(a.NB, m, decode)) {
      L.keys = reinterpret_cast<unsigned long long*>(S + (size_t)rows * ld);
      L.cnt = reinterpret_cast<int*>(L.keys + (size_t)rows * SEM_LCAP);
      L.theta = reinterpret_cast<unsigned*>(L.cnt + rows);
    }
    const SemList none{};
    if (a.events) {
      const hipError_t er = hipEventRecord(static_cast<hipEvent_t>(a.events[0]), st);
      if (er != hipSuccess) return er;
    }
    if (a.NB == 0) {
      // an empty cache: nothing to score, every list is the sink and the window
    } else if (nqc == 1) {
      if (use_list) {
        hipLaunchKernelGGL(sem_theta_kernel, dim3(a.B), dim3(SEM_THR_NT), 0, st,
                           static_cast<const unsigned short*>(a.q_idx), a.q_pos, a.n_q, i0, pg,
                           static_cast<const unsigned short*>(a.cent), a.NB, m, a.sp.n_cluster, a.p_top,
                           a.sp.select_mode == 2 ? 2 : a.sp.select_mode == 3 ? 3 : 0, L);  // 0: sampled
      }
      const int bpw = 4;
      dim3 grid((a.NB + 4 * bpw - 1) / (4 * bpw), 1, a.B);
      hipLaunchKernelGGL(sem_score_decode_kernel, grid, dim3(256), 0, st,
                         static_cast<const unsigned short*>(a.q_idx), a.q_pos, a.n_q, i0, pg,
                         static_cast<const unsigned short*>(a.cent), a.NB, m, a.sp.n_cluster, bpw, S, ld,
                         use_list ? L : none);
    } else {
      hipLaunchKernelGGL(sem_qnorm_kernel, dim3((rows + 255) / 256), dim3(256), 0, st,
                         static_cast<const unsigned short*>(a.q_idx), a.n_q, i0, nqc, rows, qn);
      constexpr int QT = 16;
      const int bpw = 4;
      dim3 grid((a.NB + 4 * bpw - 1) / (4 * bpw), (nqc + QT - 1) / QT, a.B);
      hipLaunchKernelGGL(sem_score_kernel<QT>, grid, dim3(256), 0, st, qn, a.q_pos, a.n_q, i0, nqc, pg,
                         static_cast<const unsigned short*>(a.cent), a.NB, m, a.sp.n_cluster, bpw, S, ld);
    }
    if (a.events) {
      const hipError_t er = hipEventRecord(static_cast<hipEvent_t>(a.events[1]), st);
      if (er != hipSuccess) return er;
    }
    // rows in registers: one 1024-thread workgroup per row; with enough rows to fill
    // the chip twice, a variant held to 64 VGPRs (8 waves per SIMD) runs two
    // workgroups per compute unit
    const bool many = (long long)a.B * nqc >= 512;
    auto fits = [&](int nt, int C) { return sem_fits_registers(n_max, pos_max, a.sp.n_bmax, nt, C); };
    const bool paged = pg.bt || pg.pt;
    int split = 0;
#define LSA_SEM_SEL1(NT, C, MINW, PG)  LSA_SEM_SEL2(NT, C, MINW, PG, false)
#define LSA_SEM_SEL2(NT, C, MINW, PG, LG)                                                                      \
  hipLaunchKernelGGL((sem_select_kernel<NT, C, MINW, PG, LG>), dim3(nqc, a.B), dim3(NT), 0, st, S, ld, a.q_pos,  \
                     a.n_q, i0, nqc, a.table, a.offs, a.NB, m, a.sp.n_cluster, a.sp.n_bmax, a.k, a.p_top, a.n_sink, \
                     a.n_w, W, a.idx, a.count, pg, split, LG && use_list ? L : none)
#define LSA_SEM_SEL(NT, C, MINW)           \
  do {                                     \
    if (paged)                             \
      LSA_SEM_SEL1(NT, C, MINW, true);     \
    else                                   \
      LSA_SEM_SEL1(NT, C, MINW, false);    \
  } while (0)
    if (use_list && a.NB > 0) {
      // the threshold list, ranked by the long-row selection (which takes the whole row
      // where the list missed)
      if (paged)
        LSA_SEM_SEL2(1024, 16, 1, true, true);
      else
        LSA_SEM_SEL2(1024, 16, 1, false, true);
    } else if (many && fits(1024, 4)) LSA_SEM_SEL(1024, 4, 8);
    else if (many && fits(1024, 8)) LSA_SEM_SEL(1024, 8, 8);
    else if (many && fits(512, 32)) LSA_SEM_SEL(512, 32, 4);
    else if (fits(1024, 4)) LSA_SEM_SEL(1024, 4, 1);
    else if (fits(1024, 8)) LSA_SEM_SEL(1024, 8, 1);
    else if (fits(1024, 16)) LSA_SEM_SEL(1024, 16, 1);
    else if (fits(1024, 32)) LSA_SEM_SEL(1024, 32, 1);
    else if (a.sp.n_bmax <= 64 && (n_max + SPAN_B - 1) / SPAN_B * a.p_top <= SEM_KC) {
      // long rows: spans of 16384 buckets in registers, their candidates merged; with
      // few rows the spans run as workgroups of their own (sem_span_topk_kernel), with
      // many each row's workgroup walks them
      if (a.B * nqc < 256) {
        // the last span's candidates end at most 2 * (p_top + 1) floats past its scores
        if (!sem_long_rows(a.NB, m, a.sp.n_cluster, a.sp.n_bmax) || ld < n_max + 2LL * (a.p_top + 1))
          return hipErrorInvalidValue;
        split = 1;
        const int n_spans = (int)((n_max + SPAN_B - 1) / SPAN_B);
        hipLaunchKernelGGL(sem_span_topk_kernel, dim3(n_spans, nqc, a.B), dim3(1024), 0, st, S, ld, a.q_pos,
                           a.n_q, i0, nqc, a.NB, m, a.sp.n_cluster, a.p_top);
      }
      if (paged)
        LSA_SEM_SEL2(1024, 16, 1, true, true);
      else
        LSA_SEM_SEL2(1024, 16, 1, false, true);
    } else
      hipLaunchKernelGGL(sem_select_stream_kernel, dim3(nqc, a.B), dim3(SEL_NT), 0, st, S, ld, a.q_pos, a.n_q, i0,
                         nqc, pg, a.table, a.offs, a.NB, m, a.sp.n_cluster, a.k, a.p_top, a.n_sink, a.n_w, W, a.idx,
                         a.count);
#undef LSA_SEM_SEL
#undef LSA_SEM_SEL1
#undef LSA_SEM_SEL2
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.events) {
    const hipError_t er = hipEventRecord(static_cast<hipEvent_t>(a.events[2]), st);
    if (er != hipSuccess) return er;
  }
  return hipSuccess;
}

}  // namespace lsa
