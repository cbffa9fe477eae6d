// lsa_attn.hip -- sparse attention over per-query index lists (gfx950, bf16 MFMA).
//
//     out[b,i,h,:] = sum_{j in J_i} softmax_j(scale * q[b,i,h,:] . k[b,j,:]) v[b,j,:]
// "Latent Sparse Attention (LSA)" §3.2 "Attention": attention runs only over the
// keys of J_i, one list for every query head; §2: O(k) work per query.  App. F.1
// "Attention kernels": J_i is read like a page table of single-slot pages, -1 =
// no key.  The split form (J_i cut into n_split parts merged by log-sum-exp) is
// the split-KV decode kernel the same appendix mentions.
//
// Per tile of 32 listed keys, in one wave:
//   * the 32 K rows are gathered straight into MFMA A fragments and multiplied by
//     the query's heads (B fragments, loaded once): S^T[key][head] = K Q^T with
//     v_mfma_f32_16x16x32_bf16 -- lane l then owns head (l & 15);
//   * the 32 V rows are gathered and written transposed to LDS (key pairs per
//     dword, rows padded to 18 dwords: conflict-free writes and b64 reads);
//   * fp32 online softmax in the exp2 domain (rescale of O only when a head's
//     running max moves); P goes to bf16 and is used directly as the B fragment
//     of O^T[d][head] += V^T P^T, since the lanes already hold P in the key order
//     that the A fragment (read from the transposed V tile) uses.
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

constexpr int D = 128;
constexpr int KT = 32;      // keys per tile
constexpr int RSD = 18;     // dwords per transposed V row (16 key pairs + 2 pad)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));
typedef u32 v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float xhalf32_maxf(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow16_maxf(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf32_sumf(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xrow16_sumf(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite)
__device__ __forceinline__ u32 bf16_bits(float f) {
  const u32 u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ u32 pack_bf16(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

union Frag8 {
  v8bf v;
  v4u u;
};

// LDS ordering between lanes of one wave: LDS operations of a wave complete in
// issue order, so keeping the compiler from moving them across this point is enough.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int WAVE_LDS = D * RSD;  // dwords of LDS per wave: the transposed V tile, later its partial state

// A workgroup of NW waves handles one (row, split) unit: the split's 32-key tiles are
// dealt to the waves round-robin, each wave keeps an online-softmax state for the 16
// heads, and at the end the NW states are merged through LDS.  n_split == 1 writes
// the bf16 output and LSE; otherwise a normalised fp32 partial and its LSE go to ws.
//
// Two forms.  PIPE: a wave walks many tiles with the next tile's gathers in flight
// (two register sets; rows of many queries, where the grid alone fills the chip).
// !PIPE: a wave takes at most one tile (the launch keeps the split's tiles <= NW), so
// the code is straight-line, O is born after the gathers and 16 waves fit on a CU
// (128 VGPRs) -- the split-KV decode form.  Random 256-byte row gathers reach a
// higher rate from many waves with few loads in flight each than from few waves with
// many: a wave's loads return in order, so one slow row holds back every later load
// of that wave.
template <int NW, bool PIPE>
__global__ __launch_bounds__(64 * NW, PIPE ? 2 : 16 / NW) void sparse_attn_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ idx, int n_q, long long kv_rows, long long j_lim, int H_q, int k_top,
    float scale_log2, int n_split, __bf16* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) u32 lds[NW * WAVE_LDS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const long long unit = blockIdx.x;
  const long long row = unit / n_split;
  const int split = (int)(unit % n_split);
  const int b = (int)(row / n_q);
  const int32_t* jrow = idx + row * (long long)k_top;
  // sequence b's keys: rows [b * kv_rows, b * kv_rows + j_lim) of k and v (paged caches:
  // kv_rows = 0 and the entries are rows of the shared pool)
  const __bf16* kb = k + (long long)b * kv_rows * D;
  const __bf16* vb = v + (long long)b * kv_rows * D;
  u32* vt = lds + wave * WAVE_LDS;

  // query heads as B fragments: lane (h = l&15, g) holds d = 32s + 8g .. +8 at step s.
  // Lanes of heads past H_q repeat head 0 (their results are never stored).  Loaded
  // after the first index entries and used as loaded: a wave's loads complete in
  // order, so the first gathers (which wait for the entries) do not wait for the query.
  Frag8 Qb[4];
  auto load_q = [&]() {
    const __bf16* qr = q + (row * H_q + (r16 < H_q ? r16 : 0)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) Qb[s].u = *(const v4u*)(qr + 32 * s);
  };

  v4f O[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) O[t] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  const int n_tiles = (k_top + KT - 1) / KT;
  const int t_begin = (int)((long long)n_tiles * split / n_split);
  const int t_end = (int)((long long)n_tiles * (split + 1) / n_split);
  // this wave's tiles: t_begin + wave + NW*i for i < n_my
  const int first = t_begin + wave;
  const int n_my = first < t_end ? (t_end - first + NW - 1) / NW : 0;

  // Software pipeline over the wave's tiles: index entries two tiles ahead, K/V
  // gathers one tile ahead, ping-pong register sets (no copies).  Every load is
  // unconditional, so the compiler's wait counts stay exact: a tile past the wave's
  // last one lists no key, so its gather reads one row (a single 64-byte piece per
  // load instruction), and it is not computed.
  struct Idx {
    int jA, jB, j0, j1;
  };
  struct Gat {
    Frag8 Ka[2][4];
    v4u V0[4], V1[4];
    unsigned long long vA, vB;
    bool v0ok, v1ok;
  };
  auto load_idx = [&](int i) -> Idx {
    const int base = (first + NW * min(i, n_my - 1)) * KT;
    const int none = i < n_my ? 0 : -1;
    auto e = [&](int pos) -> int { return jrow[min(pos, k_top - 1)] | (pos < k_top ? none : -1); };
    return Idx{e(base + r16), e(base + 16 + r16), e(base + 2 * r16), e(base + 2 * r16 + 1)};
  };
  auto gather = [&](Idx x, Gat& G) {
    auto ok = [&](int j) { return j >= 0 && (long long)j < j_lim; };
    G.vA = __ballot(ok(x.jA));
    G.vB = __ballot(ok(x.jB));
    // Entries without a key read the rows of a listed key of this tile instead (row 0
    // if none is listed): the score is masked to -inf and its weight set to exactly 0,
    // and the borrowed V row is replaced by zeros, so it adds nothing whatever it
    // holds.  No tile is skipped: a branch on the entries would let the compiler
    // move the tile's other loads behind the wait for them.
    int jfill = 0;
    if (G.vA | G.vB) {
      const int src = G.vA ? __ffsll((long long)G.vA) - 1 : __ffsll((long long)G.vB) - 1;
      jfill = G.vA ? __shfl(x.jA, src) : __shfl(x.jB, src);
    }
    const int jA = ok(x.jA) ? x.jA : jfill, jB = ok(x.jB) ? x.jB : jfill;
    G.v0ok = ok(x.j0);
    G.v1ok = ok(x.j1);
    const int j0 = G.v0ok ? x.j0 : jfill, j1 = G.v1ok ? x.j1 : jfill;
    // every load instruction reads whole 64-byte pieces of 16 rows
    const __bf16* ra = kb + (long long)jA * D + 8 * g;
    const __bf16* rb = kb + (long long)jB * D + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      G.Ka[0][s].u = *(const v4u*)(ra + 32 * s);
      G.Ka[1][s].u = *(const v4u*)(rb + 32 * s);
    }
    const __bf16* r0 = vb + (long long)j0 * D + 8 * g;  // rows j0 / j1, d = 8g + 32m .. +8
    const __bf16* r1 = vb + (long long)j1 * D + 8 * g;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      G.V0[m] = *(const v4u*)(r0 + 32 * m);
      G.V1[m] = *(const v4u*)(r1 + 32 * m);
    }
  };
  auto compute = [&](const Gat& G) {
    // S^T = K Q^T : lane holds keys 16*mt + 4g + i for head r16
    v4f S[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      S[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) S[mt] = mfma_bf16(G.Ka[mt][s].v, Qb[s].v, S[mt]);
    }

    // V^T into this wave's LDS tile: dword [d][kp] = (V[2kp][d], V[2kp+1][d]), d = 8g + 32m + e
    wave_lds_sync();  // previous tile's reads of vt are done
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const u32 a = G.v0ok ? G.V0[m][w2] : 0u, c = G.v1ok ? G.V1[m][w2] : 0u;
        const int d = 8 * g + 32 * m + 2 * w2;
        vt[d * RSD + r16] = __builtin_amdgcn_perm(c, a, 0x05040100u);        // low halves
        vt[(d + 1) * RSD + r16] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // high halves
      }
    }

    // online softmax (exp2 domain)
    float sv[2][4];
    float mt_max = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const unsigned long long vm = mt ? G.vB : G.vA;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * g + i;
        const bool okk = (vm >> key) & 1ull;
        sv[mt][i] = okk ? S[mt][i] * scale_log2 : -INFINITY;
        mt_max = fmaxf(mt_max, sv[mt][i]);
      }
    }
    mt_max = xhalf32_maxf(mt_max);
    mt_max = xrow16_maxf(mt_max);
    const float m_new = fmaxf(m_run, mt_max);
    if (__ballot(m_new > m_run) != 0ull) {
      const float alpha = exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) O[t2] *= alpha;
      m_run = m_new;
    }
    Frag8 Pb;
    {
      float pv[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // masked keys weigh exactly 0 (also while m_run is still -inf)
          const bool okk = ((mt ? G.vB : G.vA) >> (4 * g + i)) & 1ull;
          const float pp = okk ? exp2f(sv[mt][i] - m_run) : 0.f;
          pv[4 * mt + i] = pp;
          l_part += pp;
        }
      Pb.u = v4u{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                 pack_bf16(pv[6], pv[7])};
    }

    wave_lds_sync();  // vt written
    // O^T[d][h] += V^T[d][keys] P^T[keys][h]; A rows d = 16*dt + r16, keys 4g..4g+3, 16+4g..
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + r16;
      Frag8 Va;
      const v2u lo = *(const v2u*)(&vt[d * RSD + 2 * g]);
      const v2u hi = *(const v2u*)(&vt[d * RSD + 8 + 2 * g]);
      Va.u = v4u{lo[0], lo[1], hi[0], hi[1]};
      O[dt] = mfma_bf16(Va.v, Pb.v, O[dt]);
    }
  };

  if constexpr (PIPE) {
    if (n_my > 0) {
      Idx x0 = load_idx(0), x1 = load_idx(1);
      load_q();
      Gat G0, G1;
      gather(x0, G0);
      x0 = load_idx(2);
      for (int i = 0; i < n_my; i += 2) {
        gather(x1, G1);  // tile i+1
        x1 = load_idx(i + 3);
        compute(G0);     // tile i
        gather(x0, G0);  // tile i+2
        x0 = load_idx(i + 4);
        if (i + 1 < n_my) compute(G1);
      }
    }
  } else if (n_my > 0) {
    const Idx x = load_idx(0);
    load_q();
    __builtin_amdgcn_sched_barrier(0);  // all entries and the query in flight before the first wait
    Gat G;
    gather(x, G);
    compute(G);
  }

  // ---- merge the NW wave states through LDS: region of wave w = O[16][OSTR] | m[16] | l[16]
  // (OSTR = D + 4: the 16 head rows start 4 banks apart, so a wave's O writes do not
  // collide); the per-head weights are computed once, then each output is NW FMAs.
  constexpr int OSTR = D + 4;
  static_assert(16 * OSTR + 32 <= WAVE_LDS, "a wave's state fits its LDS region");
  float l_tot = xhalf32_sumf(l_part);
  l_tot = xrow16_sumf(l_tot);
  wave_lds_sync();
  {
    float* st = reinterpret_cast<float*>(vt);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(v4f*)(st + r16 * OSTR + 16 * dt + 4 * g) = O[dt];
    if (g == 0) {
      st[16 * OSTR + r16] = m_run;
      st[16 * OSTR + 16 + r16] = l_tot;
    }
  }
  __syncthreads();
  const float* all = reinterpret_cast<const float*>(lds);
  __shared__ float wsc[NW][16], hinv[16], hlse[16];  // per (wave, head) weight; per head 1/den, lse
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, all[w * WAVE_LDS + 16 * OSTR + h]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = all[w * WAVE_LDS + 16 * OSTR + h];
      const float sc = (M > -INFINITY && mw > -INFINITY) ? exp2f(mw - M) : 0.f;
      wsc[w][h] = sc;
      den += sc * all[w * WAVE_LDS + 16 * OSTR + 16 + h];
    }
    hinv[h] = den > 0.f ? 1.f / den : 0.f;
    hlse[h] = den > 0.f ? (M + log2f(den)) * LN2 : -INFINITY;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < H_q * D; e += 64 * NW) {
    const int h = e / D, d = e % D;
    float num = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) num += wsc[w][h] * all[w * WAVE_LDS + h * OSTR + d];
    const float o = num * hinv[h];
    if (n_split == 1) {
      reinterpret_cast<unsigned short*>(out)[(row * H_q + h) * D + d] = (unsigned short)bf16_bits(o);
      if (lse != nullptr && d == 0) lse[row * H_q + h] = hlse[h];
    } else {
      ws[(unit * H_q + h) * D + d] = o;
      if (d == 0) ws[(long long)gridDim.x * H_q * D + unit * H_q + h] = hlse[h];
    }
  }
}

// Merge of the n_split partial results of each row by log-sum-exp.  The merge is a
// handful of flops per loaded value, so its time is the latency of its loads: every
// thread owns 4 outputs of one head and issues the loads of all its splits' partials
// and LSEs before the first use (CS splits per batch of loads), and the grid spreads a
// row over H_q * D / 1024 workgroups.  Per head: M = max_s lse_s, w_s = e^(lse_s - M),
// out = (sum_s w_s x_s) / sum_s w_s, lse = M + log(sum_s w_s).
constexpr int CMB_NT = 256;  // threads per combine workgroup (4 outputs each)
constexpr int CMB_CS = 16;   // splits loaded per batch

__global__ __launch_bounds__(CMB_NT) void attn_combine_kernel(const float* __restrict__ ws, long long n_units,
                                                             int n_split, int H_q, __bf16* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int n_out = H_q * D;
  const int per_row = (n_out + 4 * CMB_NT - 1) / (4 * CMB_NT);
  const long long row = blockIdx.x / per_row;
  const int e0 = ((int)(blockIdx.x % per_row) * CMB_NT + (int)threadIdx.x) * 4;
  if (e0 >= n_out) return;
  const int h = e0 / D;
  const float* pl = ws + n_units * n_out + row * n_split * H_q + h;  // lse part of split s: pl[s * H_q]
  const float* px = ws + row * n_split * n_out + e0;                 // partial of split s: px[s * n_out]

  float M = -INFINITY, den = 0.f;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int s0, float (&ls)[CMB_CS], v4f (&x)[CMB_CS]) {
#pragma unroll
    for (int s = 0; s < CMB_CS; ++s) {
      const bool in = s0 + s < n_split;
      ls[s] = in ? pl[(s0 + s) * H_q] : -INFINITY;
      x[s] = in ? *(const v4f*)(px + (long long)(s0 + s) * n_out) : v4f{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto accumulate = [&](const float (&ls)[CMB_CS], const v4f (&x)[CMB_CS]) {
#pragma unroll
    for (int s = 0; s < CMB_CS; ++s) {
      const float w = (M > -INFINITY && ls[s] > -INFINITY) ? expf(ls[s] - M) : 0.f;
      den += w;
      acc += x[s] * w;
    }
  };
  if (n_split <= CMB_CS) {  // one batch: M from the loaded LSEs
    float ls[CMB_CS];
    v4f x[CMB_CS];
    load(0, ls, x);
#pragma unroll
    for (int s = 0; s < CMB_CS; ++s) M = fmaxf(M, ls[s]);
    accumulate(ls, x);
  } else {  // M over all splits first, then the batches
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, pl[s * H_q]);
    for (int s0 = 0; s0 < n_split; s0 += CMB_CS) {
      float ls[CMB_CS];
      v4f x[CMB_CS];
      load(s0, ls, x);
      accumulate(ls, x);
    }
  }
  acc *= den > 0.f ? 1.f / den : 0.f;
  v2u pk;
  pk[0] = pack_bf16(acc[0], acc[1]);
  pk[1] = pack_bf16(acc[2], acc[3]);
  *(v2u*)(out + row * n_out + e0) = pk;
  if (lse != nullptr && e0 % D == 0) lse[row * H_q + h] = den > 0.f ? M + logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0) return hipSuccess;
  if (a.n_split < 1 || a.n_split > 64) return hipErrorInvalidValue;  // the merges hold 64 splits
  const long long units = rows * a.n_split;
  // one (row, split) unit per workgroup; split rows whose splits hold at most 16 tiles
  // take the one-tile form with the fewest waves that give each wave one tile
  const int tiles = (a.k_top + KT - 1) / KT;
  const int per_split = (tiles + a.n_split - 1) / a.n_split;
  const long long kv_rows = a.kv_pool > 0 ? 0ll : (long long)a.L_max;
  const long long j_lim = a.kv_pool > 0 ? a.kv_pool : (long long)a.L_max;
  auto go = [&](auto kern, int nw) {
    hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(64 * nw), 0, st, (const __bf16*)a.q, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.idx, a.n_q, kv_rows, j_lim, a.H_q, a.k_top, a.scale * LOG2E, a.n_split,
                       (__bf16*)a.out, a.lse, a.ws);
  };
  if (a.n_split == 1 || per_split > 16) go(sparse_attn_kernel<ATTN_WAVES, true>, ATTN_WAVES);
  else if (per_split <= 4) go(sparse_attn_kernel<4, false>, 4);
  else if (per_split <= 8) go(sparse_attn_kernel<8, false>, 8);
  else go(sparse_attn_kernel<16, false>, 16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const long long per_row = ((long long)a.H_q * D + 4 * CMB_NT - 1) / (4 * CMB_NT);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(rows * per_row)), dim3(CMB_NT), 0, st, a.ws, units,
                     a.n_split, a.H_q, (__bf16*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace lsa
