// lsa_indexer.hip -- int8 MFMA indexer kernels for gfx950.
//
// Token scores ("Latent Sparse Attention (LSA)", §2.1 "Token Sparse Attention":
// a low-precision indexer with few heads scores every preceding key):
//     S[b,i,j] = sum_h w_h * max(0, q_idx[b,i,h,:] . k_idx[b,j,:])      (exact int32)
// Block scores of the two-stage indexer (HISA summary: block filter first; LSA
// §3.1 "Pooling": a block summary is the sum of its index keys):
//     BS[b,i,m] = sum_h w_h * max(0, q_idx[b,i,h,:] . reps[b,m,:])      (exact int64)
//
// Mapping onto the matrix cores: a query's H_I heads are the M dimension of
// v_mfma_i32_16x16x64_i8 (tiles of 16 heads), keys are N (16 per tile), d_I is K.
// Output lane l then holds heads 4*(l>>4)+e of key (l&15), so the weighted ReLU
// head sum is lane-local (v_max_i32 + v_mad_i32_i24 per element) and only the
// final sum over the four 16-lane rows crosses lanes (permlane swaps, no LDS).
#include "lsa_device.h"
#include "lsa_idx_tiles.h"
#include "lsa_internal.h"
#include "lsa_select.h"

namespace lsa {

// ---------------------------------------------------------------------------------
// Flat scores, prefill: a workgroup of NW waves, one query per wave, shares each
// 64-key tile of a span of keys through LDS.  A wave holds only its query's A
// fragments and head weights, so four waves fit on every SIMD.
//   * Key tiles travel through a ring of R register stages, issued R-1 tiles
//     ahead; the loads are unconditional (clamped past the end) and the loop is
//     unrolled by R so no stage is copied.
//   * Inside a tile the MFMAs of key group nt+1 are issued before the ReLU/weight
//     epilogue of group nt, so the matrix cores and the VALU work side by side.
//   * A tile's 64 scores end up one per lane (lane l = key l of the tile) and leave
//     as one buffer store per lane whose range check (records = the query's valid
//     keys) drops what the query may not see: no branch around a store, so the
//     memory counter the loads share with the stores stays exact.
// Slot j scores key j * stride (a stride above 1 scores an evenly spaced sample of
// the keys; slot j is valid for a query at position p iff j * stride <= p).
// SEL (thresholded selection): a wave whose row is a list row instead appends the
// (slot, score) of its scores >= the row's threshold to a buffer in LDS, and moves
// the buffer to the row's candidate list (one device atomic reserves the places)
// whenever it nears full and at the end; table rows store their scores as above.
// tile_filter (optional): only query tiles holding a row of state 2 do any work;
// row_min: only query tiles holding a row of more than row_min keys do.
// PAGED: k_idx is a pool of pages of 2^page_log2 >= 64 keys; the pool pages of the
// workgroup's keys (at most FLAT_PAGES of them: the launcher sizes the spans) are read
// into LDS first, and each key's row is looked up there.
// Grid: x = 8 * ceil(n_qtiles / 8) * n_spans (XCD-aware order, below), y = B.
constexpr int FLAT_PAGES = 4096;
template <int D, int MT, int NW, bool SEL, bool PAGED>
__global__ __launch_bounds__(64 * NW, 4) void idx_flat_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx, const int32_t* __restrict__ w,
    int w_per_query, const int32_t* __restrict__ q_pos, int n_q, int L_max, int H_I, int span,
    int n_spans, int n_qtiles, int32_t* __restrict__ scores, long long ld, int stride,
    const int32_t* __restrict__ tile_filter, int row_min, ThrArgs thr, Pages pg) {
  constexpr int KS = D / 64, KT = 64, CH = D / 16;
  constexpr int R = 3;  // register stages of key tiles
  constexpr int WBUF = 512;  // SEL: candidates a wave buffers in LDS
  static_assert(KT * CH <= 64 * NW, "one 16-byte chunk of a key tile per thread");
  __shared__ __attribute__((aligned(16))) int8_t tile[R][KT * D];
  __shared__ int wb[SEL ? NW : 1][2][WBUF];  // SEL: per wave, slots then scores

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  // Workgroups are dealt to the 8 XCDs in turn (grid.x is a multiple of 8, so
  // workgroup x runs on XCD x % 8).  XCD x takes the query tiles x, x + 8, ...
  // (longest first, interleaved so causal work balances over the XCDs) and walks them
  // span by span: the workgroups resident on one XCD at a time read the same span of
  // keys, which its L2 then serves to all of them.
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per_xcd = (n_qtiles + 7) >> 3;
  const int s = kx / per_xcd;
  const int qt_rev = (kx - s * per_xcd) * 8 + xcd;
  if (qt_rev >= n_qtiles) return;
  const int qt = n_qtiles - 1 - qt_rev;
  const int i0 = qt * NW;
  const int32_t* qp = q_pos + (long long)b * n_q;
  // last valid slot of a query at position p (-1: none)
  auto last_slot = [&](int p) { return p < 0 ? -1 : min(p, L_max - 1) / stride; };

  int pmax = -1, nmax = 0;
  bool todo = tile_filter == nullptr;
#pragma unroll
  for (int t = 0; t < NW; ++t) {
    const int i = i0 + t;
    if (i < n_q) {
      const int p = qp[i];
      pmax = max(pmax, last_slot(p));
      nmax = max(nmax, p < 0 ? 0 : min(p, L_max - 1) + 1);
      if (tile_filter != nullptr && tile_filter[(long long)b * n_q + i] == 2) todo = true;
    }
  }
  const int j_begin = s * span;
  if (j_begin > pmax || !todo || nmax <= row_min) return;
  const int j_end = min(j_begin + span, pmax + 1);

  const int i = i0 + wave;
  const bool valid = i < n_q;
  const long long row = (long long)b * n_q + (valid ? i : 0);
  const int lim = valid ? min(last_slot(qp[i]) + 1, j_end) : 0;
  const __amdgpu_buffer_rsrc_t row_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(scores + row * ld, (short)0, lim * 4, BUF_RSRC_WORD3);

  v4i A[MT][KS];
  int wt[MT][4];
  load_query<D, MT>(q_idx, w, w_per_query, row, H_I, valid, A, wt);
  // SEL: this wave's row kind and threshold (a table row, or an invalid query, keeps
  // the plain stores)
  // (kept in scalar registers: the row kind is tested once per tile)
  int list_row = 0;
  int th = 0;
  if constexpr (SEL) {
    list_row = __builtin_amdgcn_readfirstlane((valid && thr.rstate[row] == 0) ? 1 : 0);
    th = __builtin_amdgcn_readfirstlane(thr.theta[row]);
  }
  int wn = 0;  // SEL: candidates in this wave's LDS buffer (wave-uniform)
  auto flush = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int base = 0;
    if (lane == 0) base = atomicAdd(&thr.cnt[row], wn);
    base = __shfl(base, 0);
    int32_t* lsl = thr.lslot + row * thr.cap;
    int32_t* lsc = thr.lscore + row * thr.cap;
    for (int e = lane; e < wn; e += 64) {
      if (base + e < thr.cap) {
        lsl[base + e] = wb[wave][0][e];
        lsc[base + e] = wb[wave][1][e];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wn = 0;
  };

  const int8_t* kb = k_idx + (PAGED ? 0ll : (long long)b * L_max * D);
  const int n_tiles = (j_end - j_begin + KT - 1) / KT;
  const int smax = (L_max - 1) / stride;  // last slot with a key
  // thread -> (row, chunk) of the key tile; with fewer chunks than threads the extra
  // threads repeat a chunk and write the same bytes to the same place
  const int cid = tid % (KT * CH), cr = cid / CH, cc = cid % CH;
  const int tile_off = cr * D + 16 * swz<D>(cr, cc);
  __shared__ int span_pages[PAGED ? FLAT_PAGES : 1];
  int pg0 = 0;
  if constexpr (PAGED) {
    // pages of the keys gload can touch: slots j_begin .. min(j_begin + n_tiles * KT - 1, smax)
    pg0 = (int)(((long long)j_begin * stride) >> pg.page_log2);
    const int pg1 = (int)(((long long)min(j_begin + n_tiles * KT - 1, smax) * stride) >> pg.page_log2);
    const int32_t* pt = pg.page_table + (long long)b * pg.max_pages;
    for (int t = tid; t <= pg1 - pg0; t += 64 * NW) span_pages[t] = min(max(pt[pg0 + t], 0), pg.n_pages - 1);
    __syncthreads();
  }
  // Contiguous caches: a tile's keys come through a buffer resource based at the tile's
  // first key, so the only per-tile address arithmetic is scalar; a lane's offset in the
  // tile is fixed, and keys past the cache's end read as zero (the resource's range
  // check), where no stored or listed score looks.
  const long long key_bytes = (long long)L_max * D;
  const int lane_koff = cr * stride * D + 16 * cc;
  auto gload = [&](int t) -> v4i {
    const int js0 = j_begin + min(t, n_tiles - 1) * KT;
    if constexpr (PAGED) {
      const int js = min(js0 + cr, smax);
      long long key = (long long)js * stride;
      key = ((long long)span_pages[(int)(key >> pg.page_log2) - pg0] << pg.page_log2) |
            (key & ((1ll << pg.page_log2) - 1));
      return *(const v4i*)(kb + key * D + 16 * cc);
    } else {
      const long long off0 = (long long)js0 * stride * D;
      const long long rem = key_bytes - off0;  // > 0: the tile's first slot has a key
      const int n_rec = (unsigned)(rem >> 31) != 0u ? 0x7fffffff : (int)rem;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kb + off0), (short)0, n_rec, BUF_RSRC_WORD3);
      return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_koff, 0, 0));
    }
  };
  // dot products of the query's heads with the 16 keys of group nt of LDS tile buf
  auto mfmas = [&](int buf, int nt, v4i (&acc)[MT]) {
    v4i Bf[KS];
    const int r = 16 * nt + r16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      Bf[ks] = *(const v4i*)(&tile[buf][r * D + 16 * swz<D>(r, kchunk<D>(g, ks))]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma_i8(A[mt][ks], Bf[ks], acc[mt]);
    }
  };
  // this lane's share of sum_h w_h * max(0, dot_h) for its key column
  auto epilogue = [&](const v4i (&acc)[MT]) -> int {
    int ps = relu_mul24(acc[0][0], wt[0][0]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (e + mt > 0) ps = relu_mad24(acc[mt][e], wt[mt][e], ps);
    return ps;
  };
  auto compute = [&](int buf) -> int {
    int part[4];
    v4i acc0[MT], acc1[MT];
    mfmas(buf, 0, acc0);
    mfmas(buf, 1, acc1);
    part[0] = epilogue(acc0);
    mfmas(buf, 2, acc0);
    part[1] = epilogue(acc1);
    mfmas(buf, 3, acc1);
    part[2] = epilogue(acc0);
    part[3] = epilogue(acc1);
    return reduce_scatter4(part);  // lane l: key l of the tile
  };

  // R register stages and R LDS tiles: in the loop unrolled by R, tile t sits in stage
  // and LDS tile t % R = u, so every LDS address is fixed at compile time
  v4i st[R];
#pragma unroll
  for (int u = 0; u < R; ++u) st[u] = gload(u);
  *(v4i*)(&tile[0][tile_off]) = st[0];
  __syncthreads();
  const int n_pad = (n_tiles + R - 1) / R * R;
  for (int t0 = 0; t0 < n_pad; t0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = t0 + u;
      st[u] = gload(t + R);  // stage u held tile t, already in LDS
      int res = 0;
      if (t < n_tiles) res = compute(u);
      const int jt = j_begin + t * KT;  // slot of the tile's first key
      if (!SEL || list_row == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(res, row_rsrc, 4 * (jt + lane), 0, 0);
      } else {
        const bool pass = lane < lim - jt && res >= th;
        const unsigned long long bal = __builtin_amdgcn_ballot_w64(pass);
        if (bal != 0ull) {  // wave-uniform
          const int r = wn + lanes_below(bal);
          if (pass) {
            wb[wave][0][r] = jt + lane;
            wb[wave][1][r] = res;
          }
          wn += __popcll(bal);
          if (wn > WBUF - 64) flush();
        }
      }
      *(v4i*)(&tile[(u + 1) % R][tile_off]) = st[(u + 1) % R];  // tile t+1
      __syncthreads();
    }
  }
  if (SEL && list_row && wn > 0) flush();
}

// ---------------------------------------------------------------------------------
// Direct scores: one query per workgroup, each wave takes 64-slot groups and loads
// its key rows straight into MFMA B fragments (no LDS).  Used for flat rows of few
// queries (whole context split into spans over grid.x) and for the two-stage token
// stage (KEPT: slot s is key kept[s / bs] * bs + s % bs; one workgroup covers all
// slots).  The scan is bound by HBM, so each wave keeps a ring of RING groups of
// fragments: RING-1 groups of loads are in flight while one group is multiplied
// (2 waves/SIMD).
// GB (KEPT with bs a multiple of 64): a 64-slot group lies in one kept block, so one
// wave-uniform lookup of that block gives the keys of the whole group.
// Grid: x = n_spans (1 for KEPT), y = B * n_q.
template <int D, int MT, bool KEPT, bool GB>
__global__ __launch_bounds__(256, 2) void idx_direct_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx, const int32_t* __restrict__ w,
    int w_per_query, const int32_t* __restrict__ q_pos, const int32_t* __restrict__ kept, int bs,
    int n_keep, int n_q, int L_max, int H_I, int span, int32_t* __restrict__ scores, long long ld) {
  constexpr int KS = D / 64;
  constexpr int RING = 4;
  // Scores collect in LDS and leave in one burst at the end: a global store between
  // the ring's loads makes the next wait drain every load in flight (loads and stores
  // share one counter and may complete out of order).
  constexpr int SBUF = KEPT ? 8192 : DIRECT_SPAN;
  __shared__ int kept_s[KEPT ? 256 : 1];
  __shared__ __attribute__((aligned(16))) int sbuf[SBUF];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long row = blockIdx.y;
  const int b = (int)blockIdx.y / n_q;
  // Flat rows: the span's keys are loaded (clamped to the cache) and scored whatever
  // the query's position; the position only decides which scores are kept.  So the
  // position, the query and the first key groups are all requested before any of
  // them is waited for -- one memory latency at start-up instead of three.
  const int p_raw = q_pos[row];
  int p = 0, s_begin, s_lim, s_end;  // slots [s_begin, s_lim) are scored, [s_begin, s_end) kept
  if constexpr (KEPT) {
    p = min(p_raw, L_max - 1);
    if (p < 0) return;
    for (int t = tid; t < n_keep; t += 256) kept_s[t] = kept[row * n_keep + t];
    __syncthreads();
    s_begin = 0;
    s_lim = s_end = n_keep * bs;
  } else {
    s_begin = blockIdx.x * span;
    s_lim = min(s_begin + span, L_max);
    s_end = s_lim;  // narrowed to the position once it has arrived
  }

  v4i A[MT][KS];
  int wv[MT][4];
  issue_query<D, MT>(q_idx, w, w_per_query, row, H_I, A, wv);
  const int8_t* kb = k_idx + (long long)b * L_max * D;
  const long long srow = row * ld;

  // key a slot's scores come from (any slot below s_lim), and whether it is a
  // candidate of this query
  auto key_load = [&](int s) -> int {
    if constexpr (KEPT) {
      const int blk = kept_s[s / bs];  // the query's own block may run past the cache
      return blk >= 0 ? min(blk * bs + s % bs, L_max - 1) : 0;
    } else {
      return s;
    }
  };
  auto is_cand = [&](int s) -> bool {
    if (s >= s_end) return false;
    if constexpr (KEPT) {
      const int blk = kept_s[s / bs];
      return blk >= 0 && blk * bs + s % bs <= p;
    } else {
      return true;
    }
  };

  // Slots are processed in chunks of SBUF (one chunk for flat rows); the chunk's
  // scores leave LDS after its ring loop.  The ring loop is branch-free so the
  // compiler's wait counts stay exact: every wave runs the same number of iterations
  // (a multiple of RING) and loads past its last group re-read a row already in cache.
  v4i ring[RING][4][KS];
  auto load_group = [&](int c0, int c1, int i, v4i (&Bf)[4][KS]) {
    const int sg = c0 + 64 * (wave + 4 * i);
    if constexpr (GB) {
      // groups past the chunk re-read its last group (chunks are multiples of 64 slots)
      const int sgc = min(sg, c1 - 64);
      const int bi = sgc / bs;
      const int blk = kept_s[bi];
      const int k0 = (blk >= 0 ? blk * bs + (sgc - bi * bs) : 0) + r16;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int8_t* kr = kb + (long long)min(k0 + 16 * nt, L_max - 1) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kr + 16 * kchunk<D>(g, ks));
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        // a slot past the chunk (or without a kept block) reads a fallback row: its
        // score is never kept, and unconditional loads stay in flight together
        const int s = min(sg + 16 * nt + r16, c1 - 1);
        const int8_t* kr = kb + (long long)key_load(s) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kr + 16 * kchunk<D>(g, ks));
      }
    }
  };
  auto prologue = [&](int c0, int c1) {
#pragma unroll
    for (int r = 0; r < RING - 1; ++r) load_group(c0, c1, r, ring[r]);
  };
  int wt[MT][4];
  // the chunk's scores (in sbuf) to the score table
  auto store_chunk = [&](int c0, int c1) {
    if (!KEPT && (reinterpret_cast<uintptr_t>(scores + srow + c0) & 15) == 0) {
      // flat rows: the whole chunk in 16-byte non-temporal stores (scores of keys past
      // the query's position may be written: they are unspecified), which disturb the
      // key stream less than dword stores
      const int n4 = (c1 - c0) / 4;
      for (int t = tid; t < n4; t += 256)
        __builtin_nontemporal_store(*(const v4i*)&sbuf[4 * t], (v4i*)(scores + srow + c0 + 4 * t));
      for (int t = 4 * n4 + tid; t < c1 - c0; t += 256) scores[srow + c0 + t] = sbuf[t];
    } else {
      for (int t = tid; t < c1 - c0; t += 256)
        if (is_cand(c0 + t)) scores[srow + c0 + t] = sbuf[t];
    }
  };
  // the ring loop and the score flush of one chunk whose prologue has been issued
  auto run_chunk = [&](int c0, int c1) {
    const int n_groups = (c1 - c0 + 63) / 64;
    const int n_iter = ((n_groups + 3) / 4 + RING - 1) / RING * RING;  // groups per wave, padded
    auto compute_group = [&](int i, const v4i (&Bf)[4][KS]) {
      const int sg = c0 + 64 * (wave + 4 * i);
      int part[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        v4i acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] = v4i{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma_i8(A[mt][ks], Bf[nt][ks], acc[mt]);
        }
        int ps = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ps = relu_mad24(acc[mt][e], wt[mt][e], ps);
        part[nt] = ps;
      }
      const int res = reduce_scatter4(part);
      const int s = sg + 16 * g + r16;
      if (s < c1) sbuf[s - c0] = res;
    };
    for (int i0 = 0; i0 < n_iter; i0 += RING) {
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        load_group(c0, c1, i0 + r + RING - 1, ring[(r + RING - 1) % RING]);
        compute_group(i0 + r, ring[r]);
      }
    }
    __syncthreads();
    store_chunk(c0, c1);
    __syncthreads();
  };

  if constexpr (KEPT) {
    query_weights<MT>(wv, H_I, true, wt);
    for (int c0 = s_begin; c0 < s_lim; c0 += SBUF) {
      const int c1 = min(c0 + SBUF, s_lim);
      prologue(c0, c1);
      run_chunk(c0, c1);
    }
  } else {
    // the first key groups go out with the query and the position, before any wait
    prologue(s_begin, s_lim);
    query_weights<MT>(wv, H_I, true, wt);
    p = min(p_raw, L_max - 1);
    s_end = min(s_lim, p + 1);
    if (s_begin >= s_end) return;  // nothing of this span is a candidate (uniform)
    run_chunk(s_begin, s_lim);
  }
}

// ---------------------------------------------------------------------------------
// Decode scores that leave each row's selection state instead of a score table (flat
// rows of few queries, rows with more valid keys than k).  A row's n_valid keys are
// cut into gridDim.x spans of dec_span(n_valid, gridDim.x) consecutive keys, one
// 8-wave workgroup each, and the launch is sized to about one workgroup per compute
// unit: start-up and the closing selection work are paid once per compute unit, not
// once per few thousand keys.
//   * Each wave streams 64-key groups straight into MFMA B fragments through a ring
//     of RING register stages, as the direct kernel does; the groups are handed out
//     by an LDS counter as ring slots free up, so the waves finish together.
//   * The span's scores stay in LDS, and each is counted into a packed LDS histogram
//     of the selection's coarse bins (16-bit counters: a span has < 65536 keys) as it
//     is produced.
//   * At the end the workgroup finds its list's lowest bin lbw -- the highest bin such
//     that bins >= lbw hold at least min(entries, k) entries -- and writes its record
//     (DecWs): the list (its entries of bins >= lbw in slot order), its group sums, the
//     bins of its band and the header.  No span can hold k entries above the row's cut
//     bin (fewer than k entries of the whole row are), so every list reaches down to
//     the cut.  A list that would hold more than lcap entries (heavy ties in the bin
//     that completes it) is replaced by the span's slice of the score table (lbw = -1).
//     Only plain stores, issued last, which nothing waits for: no device-scope
//     atomics (several workgroups on different XCDs would contend for the row's
//     bins) and nothing to clear beforehand.
//   * PAGED: k_idx is a pool of pages of 2^page_log2 >= 64 keys; the pool pages of
//     the span are read into LDS once.  A 64-key group (spans start at multiples of
//     64) lies inside one page, so its loads are those of the contiguous layout.
// Grid: x = parts, y = B * n_q.
template <int D, int MT, bool PAGED>
__global__ __launch_bounds__(512, 1) void idx_decode_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ k_idx, const int32_t* __restrict__ w,
    int w_per_query, const int32_t* __restrict__ q_pos, int n_q, int L_max, int H_I,
    int32_t* __restrict__ scores, long long ld, DecWs sel, int k_top, Pages pg) {
  constexpr int NT = 512, NWV = NT / 64, KS = D / 64, RING = 4;
  static_assert(NGRP <= NT, "one group sum per thread");
  __shared__ __attribute__((aligned(16))) int sbuf[DEC_SPAN_MAX];
  __shared__ unsigned lh[NBINS / 2];  // bin b: 16-bit count at bit 16 * (b & 1) of word b / 2
  __shared__ int brange[2];
  __shared__ int scan_l[NWV + 1];
  __shared__ int lsh[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const long long row = blockIdx.y;
  const int part = blockIdx.x;
  const int b = (int)blockIdx.y / n_q;

  v4i A[MT][KS];
  int wv[MT][4];
  issue_query<D, MT>(q_idx, w, w_per_query, row, H_I, A, wv);
  const int n_valid = max(min(q_pos[row], L_max - 1) + 1, 0);
  // a row with no more valid keys than k takes them all: nothing to score
  if (n_valid <= k_top) return;
  const int span = dec_span(n_valid, gridDim.x);
  const int s_begin = part * span, s_end = min(s_begin + span, n_valid);
  if (s_begin >= s_end) return;  // uniform
  const int n_ent = s_end - s_begin;
  const int8_t* kb = k_idx + (PAGED ? 0ll : (long long)b * L_max * D);
  __shared__ int span_pages[PAGED ? DEC_SPAN_MAX / 64 + 2 : 1];
  const int pg0 = PAGED ? s_begin >> pg.page_log2 : 0;
  if constexpr (PAGED) {
    const int n_pg = ((s_end - 1) >> pg.page_log2) - pg0 + 1;
    const int32_t* pt = pg.page_table + (long long)b * pg.max_pages + pg0;
    for (int t = tid; t < n_pg; t += NT) span_pages[t] = min(max(pt[t], 0), pg.n_pages - 1);
    __syncthreads();
  }

  // Ring of key fragments.  Loads past the span re-read its last key, so every load
  // is unconditional.
  v4i ring[RING][4][KS];
  const int n_groups = (n_ent + 63) / 64;
  auto load_group = [&](int grp, v4i (&Bf)[4][KS]) {
    const int sg = s_begin + 64 * grp;
    // PAGED: the pool row of key j of this group is (page << page_log2) | (j & mask);
    // keys clamped to the span's last key stay in the group's page
    long long prow = 0;
    if constexpr (PAGED) prow = (long long)span_pages[(min(sg, s_end - 1) >> pg.page_log2) - pg0] << pg.page_log2;
    const int pmask = PAGED ? (1 << pg.page_log2) - 1 : -1;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int8_t* kr = kb + (prow + (min(sg + 16 * nt + r16, s_end - 1) & pmask)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) Bf[nt][ks] = *(const v4i*)(kr + 16 * kchunk<D>(g, ks));
    }
  };
  // Groups go to the waves in the order they free a ring slot: the first RING-1 of
  // each wave are fixed (wave, wave + 8, ...), the rest come from a shared counter.
  int gi[RING];  // group in each ring slot (wave-uniform)
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) {
    gi[r] = wave + NWV * r;
    load_group(gi[r], ring[r]);
  }
  __shared__ int next_grp;
  int wt[MT][4];
  query_weights<MT>(wv, H_I, true, wt);
  for (int t = tid; t < NBINS / 2; t += NT) lh[t] = 0;
  if (tid == 0) {
    brange[0] = NBINS;
    brange[1] = -1;
    next_grp = NWV * (RING - 1);
  }
  __syncthreads();

  int bmin = NBINS, bmax = -1;  // bins this thread counted into
  auto compute_group = [&](int grp, const v4i (&Bf)[4][KS]) {
    const int sg = s_begin + 64 * grp;
    int part_s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      v4i acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[mt] = mfma_i8(A[mt][ks], Bf[nt][ks], acc[mt]);
      }
      int ps = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ps = relu_mad24(acc[mt][e], wt[mt][e], ps);
      part_s[nt] = ps;
    }
    const int res = reduce_scatter4(part_s);
    const int s = sg + 16 * g + r16;
    if (s < s_end) {
      // LDS only, inside the ring loop where the waves mostly wait on HBM anyway
      sbuf[s - s_begin] = res;
      const int bin = coarse_bin(res);
      atomicAdd(&lh[bin >> 1], 1u << ((bin & 1) << 4));
      bmin = min(bmin, bin);
      bmax = max(bmax, bin);
    }
  };
  // Waves take groups from a shared counter as they free a ring slot, so a wave the
  // memory system serves faster takes more of them (with a fixed share the waves of a
  // workgroup drift far apart and the early ones idle).  A wave's groups only grow,
  // so once the oldest slot holds a group past the span, every slot does.  The grab
  // for the next slot is issued a step ahead, so its LDS latency is hidden.
  auto grab = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_grp, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int nx = grab();
  for (bool live = true; live;) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int gl = nx;
      nx = grab();
      gi[(r + RING - 1) % RING] = gl;
      load_group(gl, ring[(r + RING - 1) % RING]);
      if (gi[r] >= n_groups) {
        live = false;
        break;
      }
      compute_group(gi[r], ring[r]);
    }
  }

  // band of bins the workgroup touched (a span's scores fill a narrow band)
  for (int o = 32; o > 0; o >>= 1) {
    bmin = min(bmin, __shfl_xor(bmin, o));
    bmax = max(bmax, __shfl_xor(bmax, o));
  }
  if (lane == 0) {
    atomicMin(&brange[0], bmin);
    atomicMax(&brange[1], bmax);
  }
  __syncthreads();
  const int lo = brange[0], hi = brange[1];
  auto bin_count = [&](int bb) -> int { return (int)((lh[bb >> 1] >> ((bb & 1) << 4)) & 0xffffu); };

  // The list's lowest bin bw: thread t sums a chunk of CB bins from the top of the
  // band, a block scan finds the chunk where the count reaches need, and that thread
  // walks its chunk.
  const int need = min(n_ent, k_top);
  {
    const int CB = (hi - lo + NT) / NT;
    const int top = hi - tid * CB;  // this thread's bins: top, top-1, ..., top-CB+1 (>= lo)
    int csum = 0;
    for (int i = 0; i < CB; ++i) csum += top - i >= lo ? bin_count(top - i) : 0;
    int tot;
    const int excl = block_exclusive_scan<NT>(csum, scan_l, &tot);
    if (excl < need && excl + csum >= need) {
      int acc = excl;
      for (int i = 0; i < CB; ++i) {
        const int bb = top - i;
        const int h = bb >= lo ? bin_count(bb) : 0;
        if (acc + h >= need) {
          lsh[0] = bb;
          lsh[1] = acc + h > sel.lcap;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
  }
  const int bw = lsh[0];
  const bool tied = lsh[1] != 0;
  int n_list = 0;
  if (tied) {
    // heavy ties: the span's slice of the score table instead of a list
    int32_t* srow = scores + row * ld;
    for (int t = tid; t < n_ent; t += NT) srow[s_begin + t] = sbuf[t];
  } else {
    // The list: thread t takes C consecutive entries, reads them as 16-byte quads --
    // all reads in flight together -- and marks the selected ones in a bit mask.  C/4
    // is odd, so the lanes' first quads are an odd number of quads apart and any 16
    // lanes' quads fall in distinct bank groups (an even count, e.g. C = 64, puts
    // every lane of a read on the same banks).  A block scan of the counts gives each
    // thread its first rank, and the thread writes its entries' slots and scores in
    // slot order.
    constexpr int CQ = DEC_SPAN_MAX / NT / 4;  // quads per thread at most
    static_assert(DEC_SPAN_MAX % (4 * NT) == 0 && CQ % 2 == 1, "whole quads per thread, an odd number at most");
    constexpr int NWD = (4 * CQ + 31) / 32;
    const int thr = bin_floor(bw);  // coarse_bin(v) >= bw  <=>  v >= thr
    const int C = (((n_ent + 4 * NT - 1) / (4 * NT)) | 1) * 4;
    const int c0 = min(tid * C, n_ent), len = min(C, n_ent - c0);
    unsigned msk[NWD];  // bit j: entry c0 + j is in the list
    {
      v4i v[CQ];
#pragma unroll
      for (int q = 0; q < CQ; ++q) v[q] = *(const v4i*)&sbuf[min(c0 + 4 * q, DEC_SPAN_MAX - 4)];
#pragma unroll
      for (int wd = 0; wd < NWD; ++wd) msk[wd] = 0;
#pragma unroll
      for (int q = 0; q < CQ; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) msk[(4 * q + e) >> 5] |= (v[q][e] >= thr ? 1u : 0u) << ((4 * q + e) & 31);
#pragma unroll
      for (int wd = 0; wd < NWD; ++wd) {  // entries past the thread's own
        const int nb = len - 32 * wd;
        msk[wd] &= nb >= 32 ? ~0u : (nb <= 0 ? 0u : (1u << nb) - 1u);
      }
    }
    int cnt = 0;
#pragma unroll
    for (int wd = 0; wd < NWD; ++wd) cnt += __popc(msk[wd]);
    int r = block_exclusive_scan<NT>(cnt, scan_l, &n_list);
    int* lsl = sel.lslot(row, part);
    int* lsc = sel.lscore(row, part);
#pragma unroll
    for (int wd = 0; wd < NWD; ++wd) {
      unsigned m = msk[wd];
      while (m) {
        const int j = 32 * wd + __ffs(m) - 1;
        m &= m - 1;
        lsl[r] = s_begin + c0 + j;
        lsc[r] = sbuf[c0 + j];
        ++r;
      }
    }
  }

  // the rest of the record: group sums (thread t sums group t; skewed order, so the
  // lanes of a wave read distinct banks), the band's bins, the header
  if (tid < NGRP) {
    int sum = 0;
    if (tid * GRP <= hi && tid * GRP + GRP > lo) {
#pragma unroll
      for (int i = 0; i < GRP / 2; ++i) {
        const unsigned v = lh[tid * (GRP / 2) + ((i + tid) & (GRP / 2 - 1))];
        sum += (int)(v & 0xffffu) + (int)(v >> 16);
      }
    }
    sel.gsum(row, part)[tid] = sum;
  }
  int* hrec = sel.hist(row, part);
  for (int t = lo + tid; t <= hi; t += NT) hrec[t] = bin_count(t);
  if (tid == 0) *reinterpret_cast<int4*>(sel.hdr(row, part)) = make_int4(lo, hi, n_list, tied ? -1 : bw);
}

// ---------------------------------------------------------------------------------
// Block representatives: reps[b,m,c] = sum over the block's keys of k_idx[b,j,c].
__global__ void blk_reps_kernel(const int8_t* __restrict__ k_idx, int L_max, int D, int bs, int n_blocks,
                                long long total, int32_t* __restrict__ reps) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % D);
  const long long bm = e / D;
  const int m = (int)(bm % n_blocks);
  const long long b = bm / n_blocks;
  const int8_t* src = k_idx + (b * L_max + (long long)m * bs) * D + c;
  int acc = 0;
  for (int t = 0; t < bs; ++t) acc += src[(long long)t * D];
  reps[e] = acc;
}

// Two int8 limbs of each representative, r = 128*hi + lo with lo in [-64, 63]:
// for blocks of at most 128 int8 keys |r| <= 16384, so hi fits int8 as well.
// Row layout [hi (D bytes) | lo (D bytes)].
__global__ void blk_limbs_kernel(const int32_t* __restrict__ reps, int D, long long total,
                                 int8_t* __restrict__ limbs) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % D);
  const long long rowi = e / D;
  const int r = reps[e];
  const int hi = (r + 64) >> 7;
  const int lo = r - (hi << 7);
  limbs[rowi * 2 * D + c] = (int8_t)hi;
  limbs[rowi * 2 * D + D + c] = (int8_t)lo;
}

// Blocks of few keys (the pooled 4:1 cache): thread e owns 16-byte chunk e % (D / 16)
// of one block -- it reads that chunk of each of the block's key rows (16-byte loads,
// four rows in flight at a time), keeps the 16 byte-column sums in registers and writes
// the chunk of both limb rows with one 16-byte store each.  total = B * n_upd * D / 16.
template <int D>
__global__ __launch_bounds__(256) void blk_cache_chunks_kernel(const int8_t* __restrict__ k_idx, int L_max, int bs,
                                                               int n_blocks, int m0, int n_upd, long long total,
                                                               int8_t* __restrict__ limbs, Pages pg) {
  constexpr int CH = D / 16;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % CH);
  const long long bm = e / CH;
  const int m = m0 + (int)(bm % n_upd);
  const long long b = bm / n_upd;
  auto key_row = [&](int j) -> long long {
    if (pg.page_table == nullptr) return b * L_max + j;
    const long long page = min(max(pg.page_table[b * pg.max_pages + (j >> pg.page_log2)], 0), pg.n_pages - 1);
    return (page << pg.page_log2) | (j & ((1 << pg.page_log2) - 1));
  };
  int sum[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum[i] = 0;
  for (int t0 = 0; t0 < bs; t0 += 4) {
    v4i x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      x[u] = t0 + u < bs ? *(const v4i*)(k_idx + key_row(m * bs + t0 + u) * D + 16 * c) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum[i] += (int)(signed char)(x[u][i >> 2] >> (8 * (i & 3)));
  }
  v4i hw = v4i{0, 0, 0, 0}, lw = v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int hi = (sum[i] + 64) >> 7;
    const int lo = sum[i] - (hi << 7);
    hw[i >> 2] |= (hi & 0xff) << (8 * (i & 3));
    lw[i >> 2] |= (lo & 0xff) << (8 * (i & 3));
  }
  int8_t* dst = limbs + (b * n_blocks + m) * 2 * D + 16 * c;
  *(v4i*)dst = hw;
  *(v4i*)(dst + D) = lw;
}

// Block-key cache: blocks [m0, m0 + n_upd) of every sequence, each written as the
// two int8 limbs of its representative (the sum of its bs keys), rows laid out as
// blk_limbs_kernel writes them.  Blocks of at least BLK_CACHE_WG_MIN keys take one
// workgroup per block: thread t reads 16-byte chunk
// t % CH of every (256 / CH)-th key row of the block (all its loads issued before the
// first sum), keeps 16 column sums, and the sums of the threads sharing a chunk meet in
// LDS.  With a page table (pg.page_table set) k_idx is a pool and key j of sequence b
// is pool row page_table[b][j >> page_log2] << page_log2 | (j & mask) (page ids
// clamped).  Grid: x = B * n_upd (workgroup x: sequence x / n_upd, block m0 + x % n_upd).
constexpr int BLK_CACHE_WG_MIN = 32;
template <int D>
__global__ __launch_bounds__(256) void blk_cache_kernel(const int8_t* __restrict__ k_idx, int L_max, int bs,
                                                        int n_blocks, int m0, int n_upd,
                                                        int8_t* __restrict__ limbs, Pages pg) {
  constexpr int CH = D / 16, NG = 256 / CH, KPT = (128 + NG - 1) / NG;  // bs <= 128 keys
  __shared__ int part[NG][D + 1];
  const int tid = threadIdx.x, c = tid % CH, kg = tid / CH;
  const int m = m0 + (int)(blockIdx.x % n_upd);
  const long long b = blockIdx.x / n_upd;
  v4i x[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int t = kg + u * NG;
    x[u] = v4i{0, 0, 0, 0};
    if (t < bs) {
      const int j = m * bs + t;
      long long rowk;
      if (pg.page_table != nullptr) {
        const long long page = min(max(pg.page_table[b * pg.max_pages + (j >> pg.page_log2)], 0), pg.n_pages - 1);
        rowk = (page << pg.page_log2) | (j & ((1 << pg.page_log2) - 1));
      } else {
        rowk = b * L_max + j;
      }
      x[u] = *(const v4i*)(k_idx + rowk * D + 16 * c);
    }
  }
  int sum[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum[i] = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum[i] += (int)(signed char)(x[u][i >> 2] >> (8 * (i & 3)));
#pragma unroll
  for (int i = 0; i < 16; ++i) part[kg][16 * c + i] = sum[i];
  __syncthreads();
  if (tid < D) {
    int r = 0;
#pragma unroll 8
    for (int g2 = 0; g2 < NG; ++g2) r += part[g2][tid];
    const int hi = (r + 64) >> 7;
    int8_t* dst = limbs + (b * n_blocks + m) * 2 * D;
    dst[tid] = (int8_t)hi;
    dst[D + tid] = (int8_t)(r - (hi << 7));
  }
}

// Block scores with the flat kernel's tiling: the "keys" are block limb rows of
// 2*D bytes; q.r = 128*(q.hi) + (q.lo) is exact in int32 (|q.r| < 2^29), then
// ReLU and the weighted head sum accumulate in int64.  Block m is scored for a
// query iff m < floor(q_pos / bs) (its own block is never scored).
// stride > 1 scores only blocks 0, stride, 2 stride, ... (column m of a row holds
// block m * stride): the thresholded keep's sample.  MODE 0 writes every scored block
// to the table.  MODE 1 (thresholded scan) writes table rows (state 1) to the table and
// appends each list row's blocks whose score reaches its threshold to its list: one
// atomic per wave, query and tile reserves the slots, and the tile's entries are
// written after the next tile's products, so the atomic's round trip hides behind
// them.  MODE 2 scores the tiles of the fallback list (tiles holding a row in state 2)
// and writes only those rows, on a grid of BLK_THR_FB_SLOTS x n_spans workgroups.
// Grid (MODE 0, 1): x = 8 * ceil(n_qtiles / 8) * n_spans (the flat kernel's XCD-aware
// order), y = B.
template <int D, int MT, int QW, int MODE>
__global__ __launch_bounds__(256, 2) void blk_scores_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ limbs, const int32_t* __restrict__ w,
    int w_per_query, const int32_t* __restrict__ q_pos, int n_q, int n_blocks, int L_max, int H_I,
    int bs, int span, int n_spans, int n_qtiles, long long* __restrict__ bscores, long long ld, int stride,
    BlkThr thr) {
  static_assert(QW == 2, "reduce_scatter8_64 assumes two queries per wave");
  constexpr int KS = D / 64, KT = 64, QT = 4 * QW, RB = 2 * D, CH = RB / 16;
  constexpr int LOADS = KT * CH / 256;
  static_assert(QT == BLK_THR_QT, "the fallback list's tiles");
  __shared__ __attribute__((aligned(16))) int8_t tile[2][KT * RB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int nv = (n_blocks + stride - 1) / stride;  // columns: blocks 0, stride, ...
  // columns [0, own_col(p)) are scored for a query at position p
  auto own_col = [&](int pp) { return (min(pp / bs, n_blocks) + stride - 1) / stride; };

  // query tile qt of sequence b over span s of columns
  auto body = [&](int b, int qt, int s) {
    const int i0 = qt * QT;
    const int32_t* qp = q_pos + (long long)b * n_q;
    // MODE 2: rows in state 2 only
    auto takes = [&](int i) { return MODE != 2 || thr.rstate[(long long)b * n_q + i] == 2; };
    int omax = 0;  // columns [0, omax) are scored for some query of the tile
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int i = i0 + t;
      if (i < n_q) {
        const int pp = min(qp[i], L_max - 1);
        if (pp >= 0 && takes(i)) omax = max(omax, own_col(pp));
      }
    }
    const int m_begin = s * span;
    if (m_begin >= omax) return;
    const int m_end = min(m_begin + span, omax);

    v4i A[QW][MT][KS];
    int wt[QW][MT][4];
    int own[QW];
    long long srow[QW];
    long long rid[QW];  // flattened row
    long long th[QW];   // MODE 1: threshold of a list row
    bool lst[QW];       // MODE 1: the row appends to its list
#pragma unroll
    for (int q = 0; q < QW; ++q) {
      const int i = i0 + wave * QW + q;
      const bool valid = i < n_q;
      const long long row = (long long)b * n_q + (valid ? i : 0);
      const int pp = valid ? min(qp[i], L_max - 1) : -1;
      own[q] = pp >= 0 && takes(i) ? own_col(pp) : 0;
      srow[q] = row * ld;
      rid[q] = row;
      th[q] = 0;
      lst[q] = false;
      if constexpr (MODE == 1) {
        if (valid && pp >= 0 && thr.rstate[row] == 0) {
          lst[q] = true;
          th[q] = thr.theta[row];
        }
      }
      load_query<D, MT>(q_idx, w, w_per_query, row, H_I, valid, A[q], wt[q]);
    }

    // Column rows come through buffer resources based at the rows a load instruction
    // starts on, so the per-tile address arithmetic is scalar; a lane's offset is fixed,
    // and columns past the last block read as zero (the resource's range check), where
    // no stored or listed score looks.
    const int8_t* lb = limbs + (long long)b * n_blocks * RB;
    // (n_blocks <= 65536 rows of RB bytes: every offset here fits in 32 bits)
    const int limb_bytes = n_blocks * RB;
    const int lane_loff = (tid / CH) * stride * RB + 16 * (tid % CH);
    v4i stage[LOADS];
    auto gload = [&](int m0) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int off0 = (m0 + u * (256 / CH)) * stride * RB;  // row of thread 0
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(lb + off0), (short)0, max(limb_bytes - off0, 0), BUF_RSRC_WORD3);
        stage[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_loff, 0, 0));
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int cid = tid + 256 * u, r = cid / CH, c = cid % CH;
        *(v4i*)(&tile[buf][r * RB + 16 * swz<RB>(r, c)]) = stage[u];
      }
    };

    // lanes 0-31 hold query 0 of the wave, lanes 32-63 query 1
    const int lq = g >> 1;
    const unsigned long long half = lq ? 0xFFFFFFFF00000000ull : 0x00000000FFFFFFFFull;
    // MODE 1: the previous tile's entries waiting for their slots
    long long pv[2] = {0, 0};
    int pm[2] = {0, 0};
    unsigned long long pb[2] = {0ull, 0ull};
    int psb = 0;
    auto flush = [&]() {
      const int sb = __shfl(psb, lane & 32);
      const long long row = lq ? rid[1] : rid[0];
      const int n0 = __popcll(pb[0]);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (!((pb[e] >> lane) & 1ull)) continue;
        const int slot = sb + (e ? n0 + lanes_below(pb[1]) : lanes_below(pb[0]));
        if (slot < thr.cap) {
          thr.lblk[row * thr.cap + slot] = pm[e];
          thr.lscore[row * thr.cap + slot] = pv[e];
        }
      }
    };

    const int n_tiles = (m_end - m_begin + KT - 1) / KT;
    gload(m_begin);
    swrite(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int m0 = m_begin + t * KT;
      const int buf = t & 1;
      if (t + 1 < n_tiles) gload(m0 + KT);
      long long part[8];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        v4i Bh[KS], Bl[KS];
        const int r = 16 * nt + r16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = kchunk<D>(g, ks);
          Bh[ks] = *(const v4i*)(&tile[buf][r * RB + 16 * swz<RB>(r, c)]);
          Bl[ks] = *(const v4i*)(&tile[buf][r * RB + 16 * swz<RB>(r, c + D / 16)]);
        }
#pragma unroll
        for (int q = 0; q < QW; ++q) {
          long long ps = 0;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            v4i ah = v4i{0, 0, 0, 0}, al = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              ah = mfma_i8(A[q][mt][ks], Bh[ks], ah);
              al = mfma_i8(A[q][mt][ks], Bl[ks], al);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int x = (ah[e] << 7) + al[e];
              ps = (mt == 0 && e == 0) ? relu_mul64(x, wt[q][mt][e]) : relu_mad64(x, wt[q][mt][e], ps);
            }
          }
          part[4 * q + nt] = ps;
        }
      }
      long long res[2];
      reduce_scatter8_64(part, res);
      {
        const int o = lq ? own[1] : own[0];
        const long long base = lq ? srow[1] : srow[0];
        if constexpr (MODE == 1) {
          if (t > 0) flush();
          const bool ls = lq ? lst[1] : lst[0];
          const long long tq = lq ? th[1] : th[0];
          bool pass[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int m = m0 + 16 * (2 * (g & 1) + e) + r16;
            pass[e] = ls && m < o && res[e] >= tq;
            if (!ls && m < o) bscores[base + m] = res[e];
            pv[e] = res[e];
            pm[e] = m;
          }
          pb[0] = __ballot(pass[0]) & half;
          pb[1] = __ballot(pass[1]) & half;
          const int n = __popcll(pb[0]) + __popcll(pb[1]);
          psb = 0;
          if ((lane & 31) == 0 && n > 0) psb = atomicAdd(&thr.cnt[lq ? rid[1] : rid[0]], n);
        } else {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int m = m0 + 16 * (2 * (g & 1) + e) + r16;
            if (m < o) bscores[base + m] = res[e];
          }
        }
      }
      if (t + 1 < n_tiles) swrite(buf ^ 1);
      __syncthreads();
    }
    if constexpr (MODE == 1) {
      if (n_tiles > 0) flush();
    }
  };

  if constexpr (MODE == 2) {
    // the listed tiles, BLK_THR_FB_SLOTS at a time
    const int s = blockIdx.x % n_spans;
    const int n_fb = *thr.tcnt;
    for (int j = blockIdx.x / n_spans; j < n_fb; j += BLK_THR_FB_SLOTS) {
      const int tl = thr.tlist[j];
      body(tl / n_qtiles, tl % n_qtiles, s);
      __syncthreads();
    }
  } else {
    // Workgroups are dealt to the 8 XCDs in turn (grid.x is a multiple of 8, so
    // workgroup x runs on XCD x % 8).  XCD x takes the query tiles x, x + 8, ...
    // (longest first, interleaved so causal work balances over the XCDs) and walks them
    // span by span: the workgroups resident on one XCD at a time read the same span of
    // keys, which its L2 then serves to all of them.
    const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
    const int per_xcd = (n_qtiles + 7) >> 3;
    const int s = kx / per_xcd;
    const int qt_rev = (kx - s * per_xcd) * 8 + xcd;
    if (qt_rev >= n_qtiles) return;
    body(blockIdx.y, n_qtiles - 1 - qt_rev, s);
  }
}

// ---------------------------------------------------------------------------------
// Block scores of decode-shaped rows (few queries per sequence, many blocks): one
// query per workgroup of 4 waves and a span of its blocks; each wave streams 32-block
// groups of block-key rows (hi, lo parts) straight into MFMA B fragments through a
// ring of RING register stages (loads unconditional, clamped to the span's last
// block), as the flat decode scan does with index keys.  Per block: the two dot
// products give q.r = 128 (q.hi) + q.lo exactly in int32, then ReLU and the weighted
// head sum in int64; the sum over the four 16-lane rows ends with one value per block
// in lanes of rows 0 and 2.  Blocks m < own = min(floor(q_pos / bs), n_blocks) are
// scored.  The span's scores collect in LDS (span <= BLK_DEC_SPAN) and leave in one
// burst at the end: a store between the ring's loads would make the next wait drain
// the loads in flight (loads and stores share one counter).
// With cand.key set, the workgroup instead keeps its span's best min(n_keep - 1, its
// blocks) by (score desc, block asc) -- every block the row keeps from this span is
// among them -- and writes those candidates (BlkCand) in block order: a few KB per
// span instead of the span's scores.
// Grid: x = spans, y = B * n_q.
constexpr int BLK_DEC_SPAN = 4096;
template <int D, int MT>
__global__ __launch_bounds__(256, 2) void blk_decode_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ limbs, const int32_t* __restrict__ w,
    int w_per_query, const int32_t* __restrict__ q_pos, int n_q, int n_blocks, int H_I, int bs, int span,
    long long* __restrict__ bscores, long long ld, BlkCand cand, int n_keep) {
  constexpr int KS = D / 64, RB = 2 * D, RING = 4, GB = 32;  // GB blocks per group
  __shared__ __attribute__((aligned(16))) long long sbuf[BLK_DEC_SPAN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const long long row = blockIdx.y;
  const int b = (int)(row / n_q);
  v4i A[MT][KS];
  int wv[MT][4];
  issue_query<D, MT>(q_idx, w, w_per_query, row, H_I, A, wv);
  const int p = q_pos[row];
  if (p < 0) return;
  const int own = min(p / bs, n_blocks);
  const int m_begin = blockIdx.x * span, m_end = min(m_begin + span, own);
  if (m_begin >= m_end) return;  // uniform
  const int8_t* lb = limbs + (long long)b * n_blocks * RB;
  const int n_groups = (m_end - m_begin + GB - 1) / GB;
  // this wave's groups: wave, wave + 4, ...; padded to a multiple of RING (the extra
  // loads re-read the span's last block and are not computed)
  const int n_my = wave < n_groups ? (n_groups - wave + 3) / 4 : 0;
  const int n_iter = (n_my + RING - 1) / RING * RING;
  v4i ring[RING][2][2][KS];  // [stage][nt][part][ks]
  auto load_group = [&](int i, v4i (&Bf)[2][2][KS]) {
    const int sg = m_begin + GB * (wave + 4 * i);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int8_t* br = lb + (long long)min(sg + 16 * nt + r16, m_end - 1) * RB;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Bf[nt][h][ks] = *(const v4i*)(br + h * D + 16 * kchunk<D>(g, ks));
    }
  };
#pragma unroll
  for (int r = 0; r < RING - 1; ++r) load_group(r, ring[r]);
  int wt[MT][4];
  query_weights<MT>(wv, H_I, true, wt);
  auto compute_group = [&](int i, const v4i (&Bf)[2][2][KS]) {
    long long part[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      long long ps = 0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v4i ah = v4i{0, 0, 0, 0}, al = v4i{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ah = mfma_i8(A[mt][ks], Bf[nt][0][ks], ah);
          al = mfma_i8(A[mt][ks], Bf[nt][1][ks], al);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) ps = relu_mad64((ah[e] << 7) + al[e], wt[mt][e], ps);
      }
      part[nt] = ps;
    }
    // rows 0, 1 of the lower half end with block (nt 0, r16); rows 2, 3 with (nt 1, r16)
    const long long hsum = xhalf32_sum64(part[0], part[1]);
    const long long tot = xrow16_sum64(hsum, hsum);
    const int m = m_begin + GB * (wave + 4 * i) + 16 * (g >> 1) + r16;
    if ((g & 1) == 0 && m < m_end) sbuf[m - m_begin] = tot;
  };
  for (int i0 = 0; i0 < n_iter; i0 += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int i = i0 + r;
      load_group(min(i + RING - 1, n_my - 1), ring[(r + RING - 1) % RING]);
      if (i < n_my) compute_group(i, ring[r]);
    }
  }
  __syncthreads();
  if (cand.key == nullptr) {
    long long* srow = bscores + row * ld + m_begin;
    for (int t = tid; t < m_end - m_begin; t += 256) srow[t] = sbuf[t];
    return;
  }
  // the span's candidates: keys (score with the sign bit flipped: unsigned order) in
  // registers, position c * 256 + tid = block m_begin + position
  constexpr int CK = BLK_DEC_SPAN / 256;
  __shared__ int hist[2048];
  __shared__ unsigned bm[BLK_DEC_SPAN / 32], eqm[BLK_DEC_SPAN / 32];
  __shared__ int scan_tmp[5], sh[2];
  __shared__ unsigned long long shu[2];
  const int n_e = m_end - m_begin;
  unsigned long long key[CK];
  unsigned vmask = 0u;
#pragma unroll
  for (int c = 0; c < CK; ++c) {
    const int pos = c * 256 + tid;
    key[c] = pos < n_e ? (unsigned long long)sbuf[pos] ^ 0x8000000000000000ull : 0ull;
    vmask |= (pos < n_e ? 1u : 0u) << c;
  }
  const int need = min(min(n_keep - 1, own), n_e);
  unsigned long long T = 0ull;  // need >= n_e: every block of the span
  int need_eq = n_e;
  if (need < n_e) T = radix_cut64<256, CK>(key, vmask, need, hist, scan_tmp, sh, shu, &need_eq);
  mark_kept64<256, CK>(key, vmask, T, need_eq, bm, eqm, scan_tmp);
  const long long base = (row * cand.spans + blockIdx.x) * (long long)cand.cap;
  const int n_out = emit_marked<256>(bm, BLK_DEC_SPAN / 32, scan_tmp, [&](int r, int pos) {
    if (r < cand.cap) {
      cand.key[base + r] = sbuf[pos];
      cand.blk[base + r] = m_begin + pos;
    }
  });
  if (tid == 0) cand.cnt[row * cand.spans + blockIdx.x] = min(n_out, cand.cap);
}

// ---------------------------------------------------------------------------------
// host-side launchers
template <int D, int MT>
static hipError_t launch_flat_t(const IdxArgs& a, hipStream_t st) {
  constexpr int NW = 8;  // queries (= waves) per workgroup
  const int stride = a.stride > 1 ? a.stride : 1;
  const int n_qtiles = (a.n_q + NW - 1) / NW;
  const int n_slots = (a.L_max - 1) / stride + 1;
  const bool paged = a.pages.page_table != nullptr;
  int span = a.span;
  if (paged) {
    if (a.pages.page_log2 < 6 || a.pages.n_pages < 1 || (long long)a.pages.max_pages << a.pages.page_log2 < a.L_max)
      return hipErrorInvalidValue;
    // a workgroup's keys span at most FLAT_PAGES pages
    const long long fit = ((long long)(FLAT_PAGES - 2) << a.pages.page_log2) / stride / 64 * 64;
    if (fit < 64) return hipErrorInvalidValue;
    span = (int)std::min<long long>(span, fit);
  }
  const int n_spans = (n_slots + span - 1) / span;
  dim3 grid((unsigned)(8 * ((n_qtiles + 7) / 8) * n_spans), (unsigned)a.B);
  const bool sel = a.thr.theta != nullptr;
  if (sel && (a.thr.rstate == nullptr || a.thr.cnt == nullptr || a.thr.lslot == nullptr || a.thr.lscore == nullptr ||
              a.thr.cap < 1))
    return hipErrorInvalidValue;
#define LSA_FLAT(SEL, PG)                                                                                         \
  hipLaunchKernelGGL((idx_flat_kernel<D, MT, NW, SEL, PG>), grid, dim3(64 * NW), 0, st, a.q_idx, a.k_idx, a.w,     \
                     a.w_per_query, a.q_pos, a.n_q, a.L_max, a.H_I, span, n_spans, n_qtiles, a.scores,             \
                     (long long)a.ld, stride, a.tile_filter, a.row_min, a.thr, a.pages)
  if (sel) {
    if (paged) LSA_FLAT(true, true);
    else LSA_FLAT(true, false);
  } else {
    if (paged) LSA_FLAT(false, true);
    else LSA_FLAT(false, false);
  }
#undef LSA_FLAT
  return hipGetLastError();
}
template <int D, int MT, bool KEPT>
static hipError_t launch_direct_t(const IdxArgs& a, hipStream_t st) {
  if (a.sel_base != nullptr) {
    // decode rows that build their selection state: one span per workgroup, the
    // span lists in the layout the per-row finish reads
    if (KEPT || a.sel_parts < 1 || a.sel_parts > DEC_MAX_PARTS || a.sel_lcap < 1 ||
        dec_span(a.L_max, a.sel_parts) > DEC_SPAN_MAX)
      return hipErrorInvalidValue;
    DecWs sel;
    sel.base = a.sel_base;
    sel.rec_ints = a.sel_rec_ints;
    sel.parts = a.sel_parts;
    sel.lcap = a.sel_lcap;
    const dim3 grid((unsigned)a.sel_parts, (unsigned)(a.B * a.n_q));
    if (a.pages.page_table != nullptr) {
      if (a.pages.page_log2 < 6 || a.pages.page_log2 > 30 || a.pages.n_pages < 1 ||
          (long long)a.pages.max_pages << a.pages.page_log2 != a.L_max)
        return hipErrorInvalidValue;
      hipLaunchKernelGGL((idx_decode_kernel<D, MT, true>), grid, dim3(512), 0, st, a.q_idx, a.k_idx, a.w,
                         a.w_per_query, a.q_pos, a.n_q, a.L_max, a.H_I, a.scores, (long long)a.ld, sel, a.k_top,
                         a.pages);
    } else {
      hipLaunchKernelGGL((idx_decode_kernel<D, MT, false>), grid, dim3(512), 0, st, a.q_idx, a.k_idx, a.w,
                         a.w_per_query, a.q_pos, a.n_q, a.L_max, a.H_I, a.scores, (long long)a.ld, sel, a.k_top,
                         a.pages);
    }
    return hipGetLastError();
  }
  // flat rows: one span per workgroup, exactly the LDS score buffer
  if (!KEPT && a.span != DIRECT_SPAN) return hipErrorInvalidValue;
  const int n_spans = KEPT ? 1 : (a.L_max + a.span - 1) / a.span;
  dim3 grid((unsigned)n_spans, (unsigned)(a.B * a.n_q));
  if (KEPT && a.block_size % 64 == 0)
    hipLaunchKernelGGL((idx_direct_kernel<D, MT, KEPT, KEPT>), grid, dim3(256), 0, st, a.q_idx, a.k_idx, a.w,
                       a.w_per_query, a.q_pos, a.kept, a.block_size, a.n_keep, a.n_q, a.L_max, a.H_I, a.span,
                       a.scores, (long long)a.ld);
  else
    hipLaunchKernelGGL((idx_direct_kernel<D, MT, KEPT, false>), grid, dim3(256), 0, st, a.q_idx, a.k_idx, a.w,
                       a.w_per_query, a.q_pos, a.kept, a.block_size, a.n_keep, a.n_q, a.L_max, a.H_I, a.span,
                       a.scores, (long long)a.ld);
  return hipGetLastError();
}

#define LSA_DISPATCH_MT(H, CALL)            \
  switch (((H) + 15) / 16) {                \
    case 1: return CALL(1);                 \
    case 2: return CALL(2);                 \
    case 3: return CALL(3);                 \
    case 4: return CALL(4);                 \
    default: return hipErrorInvalidValue;   \
  }

hipError_t launch_index_scores(const IdxArgs& a, hipStream_t st) {
  // paged caches: the decode selection and the flat prefill kernel
  if (a.pages.page_table != nullptr && (a.kept != nullptr || (a.use_direct && a.sel_base == nullptr)))
    return hipErrorInvalidValue;
  const bool kept = a.kept != nullptr;
  const bool direct = kept || a.use_direct;
  if (a.d_I == 128) {
    if (kept) {
#define C(MT) launch_direct_t<128, MT, true>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    } else if (direct) {
#define C(MT) launch_direct_t<128, MT, false>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    } else {
#define C(MT) launch_flat_t<128, MT>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    }
  } else {
    if (kept) {
#define C(MT) launch_direct_t<64, MT, true>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    } else if (direct) {
#define C(MT) launch_direct_t<64, MT, false>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    } else {
#define C(MT) launch_flat_t<64, MT>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    }
  }
}

hipError_t launch_block_reps(const int8_t* k_idx, int B, int L_max, int d_I, int bs, int n_blocks,
                             int32_t* reps, hipStream_t st) {
  const long long total = (long long)B * n_blocks * d_I;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(blk_reps_kernel, dim3(blocks), dim3(256), 0, st, k_idx, L_max, d_I, bs, n_blocks,
                     total, reps);
  return hipGetLastError();
}

hipError_t launch_block_limbs(const int32_t* reps, int B, int n_blocks, int d_I, int8_t* limbs,
                              hipStream_t st) {
  const long long total = (long long)B * n_blocks * d_I;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(blk_limbs_kernel, dim3(blocks), dim3(256), 0, st, reps, d_I, total, limbs);
  return hipGetLastError();
}

hipError_t launch_block_cache(const int8_t* k_idx, int B, int L_max, int d_I, int bs, int n_blocks, int m0,
                              int n_upd, int8_t* limbs, hipStream_t st, const Pages& pg) {
  const long long total = (long long)B * n_upd * d_I;
  if (total == 0) return hipSuccess;
  if (m0 < 0 || n_upd < 0 || m0 + n_upd > n_blocks || (long long)(m0 + n_upd) * bs > L_max) return hipErrorInvalidValue;
  if (pg.page_table != nullptr &&
      (pg.page_log2 < 6 || pg.page_log2 > 30 || pg.n_pages < 1 || (long long)pg.max_pages << pg.page_log2 < L_max))
    return hipErrorInvalidValue;
  if (bs < 1 || bs > 128 || (d_I != 64 && d_I != 128)) return hipErrorInvalidValue;
  if (bs < BLK_CACHE_WG_MIN) {
    const long long chunks = total / 16;  // one thread per 16-byte chunk of a block
    if ((chunks + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((chunks + 255) / 256));
    if (d_I == 128)
      hipLaunchKernelGGL(blk_cache_chunks_kernel<128>, grid, dim3(256), 0, st, k_idx, L_max, bs, n_blocks, m0, n_upd,
                         chunks, limbs, pg);
    else
      hipLaunchKernelGGL(blk_cache_chunks_kernel<64>, grid, dim3(256), 0, st, k_idx, L_max, bs, n_blocks, m0, n_upd,
                         chunks, limbs, pg);
    return hipGetLastError();
  }
  if (total / d_I > 0x7fffffffLL) return hipErrorInvalidValue;
  if (d_I == 128)
    hipLaunchKernelGGL(blk_cache_kernel<128>, dim3((unsigned)(total / d_I)), dim3(256), 0, st, k_idx, L_max, bs,
                       n_blocks, m0, n_upd, limbs, pg);
  else
    hipLaunchKernelGGL(blk_cache_kernel<64>, dim3((unsigned)(total / d_I)), dim3(256), 0, st, k_idx, L_max, bs,
                       n_blocks, m0, n_upd, limbs, pg);
  return hipGetLastError();
}

template <int D, int MT>
static hipError_t launch_blk_scores_t(const BlkArgs& a, hipStream_t st) {
  const int QT = 8;
  const int n_qtiles = (a.n_q + QT - 1) / QT;
  const int span = a.span;
  if (a.mode < 0 || a.mode > 2 || (a.mode != 0 && (a.thr.rstate == nullptr || a.stride > 1)) ||
      (a.mode == 1 && (a.thr.theta == nullptr || a.thr.cnt == nullptr || a.thr.lblk == nullptr ||
                       a.thr.lscore == nullptr || a.thr.cap < 1)) ||
      (a.mode == 2 && (a.thr.tlist == nullptr || a.thr.tcnt == nullptr)))
    return hipErrorInvalidValue;
  // columns: blocks 0, stride, 2 stride, ...
  const int n_cols = a.stride > 1 ? (a.n_blocks + a.stride - 1) / a.stride : a.n_blocks;
  const int n_spans = (n_cols + span - 1) / span;
  if (n_spans == 0) return hipSuccess;
  // the kernel's XCD-aware order: 8 XCDs x ceil(n_qtiles / 8) query tiles x n_spans
  dim3 grid((unsigned)(8 * ((n_qtiles + 7) / 8) * n_spans), (unsigned)a.B);
  const int stride = a.stride > 1 ? a.stride : 1;
  if (a.mode == 0)
    hipLaunchKernelGGL((blk_scores_kernel<D, MT, 2, 0>), grid, dim3(256), 0, st, a.q_idx, a.limbs, a.w,
                       a.w_per_query, a.q_pos, a.n_q, a.n_blocks, a.L_max, a.H_I, a.block_size, span,
                       n_spans, n_qtiles, a.bscores, (long long)a.ld, stride, a.thr);
  else if (a.mode == 1)
    hipLaunchKernelGGL((blk_scores_kernel<D, MT, 2, 1>), grid, dim3(256), 0, st, a.q_idx, a.limbs, a.w,
                       a.w_per_query, a.q_pos, a.n_q, a.n_blocks, a.L_max, a.H_I, a.block_size, span,
                       n_spans, n_qtiles, a.bscores, (long long)a.ld, 1, a.thr);
  else
    hipLaunchKernelGGL((blk_scores_kernel<D, MT, 2, 2>), dim3((unsigned)(BLK_THR_FB_SLOTS * n_spans)), dim3(256), 0,
                       st, a.q_idx, a.limbs, a.w, a.w_per_query, a.q_pos, a.n_q, a.n_blocks, a.L_max, a.H_I,
                       a.block_size, span, n_spans, n_qtiles, a.bscores, (long long)a.ld, 1, a.thr);
  return hipGetLastError();
}

// Spans of the decode-shaped block scoring: about 512 workgroups in all (two per compute
// unit, all resident at once), spans of at least 512 blocks and at most BLK_DEC_SPAN.
static int blk_decode_span(long long rows, int n_blocks) {
  long long want = std::max(1ll, std::min((512 + rows - 1) / rows, (long long)(n_blocks + 511) / 512));
  want = std::max(want, (long long)(n_blocks + BLK_DEC_SPAN - 1) / BLK_DEC_SPAN);  // spans fit the LDS buffer
  return (int)std::min<long long>(((n_blocks + want - 1) / want + 31) / 32 * 32, BLK_DEC_SPAN);
}

bool blk_cand_layout(long long rows, int n_q, int n_blocks, int n_keep, void* region, size_t region_bytes,
                     BlkCand* c) {
  if (n_q >= 8 || rows <= 0 || n_blocks <= 0 || n_keep < 2 || region == nullptr) return false;
  c->span = blk_decode_span(rows, n_blocks);
  c->spans = (n_blocks + c->span - 1) / c->span;
  c->cap = n_keep - 1;
  // the merge holds a row's candidates in registers of one workgroup: at most 8 per thread
  if ((long long)c->spans * c->cap > 8 * 1024) return false;
  const size_t n = (size_t)rows * c->spans * c->cap;
  const size_t bytes = n * 8 + n * 4 + (size_t)rows * c->spans * 4;
  if (bytes > region_bytes || (reinterpret_cast<uintptr_t>(region) & 7) != 0) return false;
  c->key = static_cast<long long*>(region);
  c->blk = reinterpret_cast<int*>(c->key + n);
  c->cnt = c->blk + n;
  return true;
}

template <int D, int MT>
static hipError_t launch_blk_decode_t(const BlkArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_q;
  if (rows == 0 || a.n_blocks <= 0) return hipSuccess;  // no complete block to score
  const int span = a.cand.key != nullptr ? a.cand.span : blk_decode_span(rows, a.n_blocks);
  const int n_spans = (a.n_blocks + span - 1) / span;
  if (a.cand.key != nullptr && (n_spans != a.cand.spans || span > BLK_DEC_SPAN)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((blk_decode_kernel<D, MT>), dim3((unsigned)n_spans, (unsigned)rows), dim3(256), 0, st,
                     a.q_idx, a.limbs, a.w, a.w_per_query, a.q_pos, a.n_q, a.n_blocks, a.H_I, a.block_size, span,
                     a.bscores, a.ld, a.cand, a.cand.cap + 1);
  return hipGetLastError();
}

hipError_t launch_block_scores(const BlkArgs& a, hipStream_t st) {
  if (a.n_q < 8) {  // decode-shaped rows: one query per workgroup
    if (a.mode != 0 || a.stride > 1) return hipErrorInvalidValue;  // prefill-shaped rows only
    if (a.d_I == 128) {
#define C(MT) launch_blk_decode_t<128, MT>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    } else {
#define C(MT) launch_blk_decode_t<64, MT>(a, st)
      LSA_DISPATCH_MT(a.H_I, C)
#undef C
    }
  }
  if (a.d_I == 128) {
#define C(MT) launch_blk_scores_t<128, MT>(a, st)
    LSA_DISPATCH_MT(a.H_I, C)
#undef C
  } else {
#define C(MT) launch_blk_scores_t<64, MT>(a, st)
    LSA_DISPATCH_MT(a.H_I, C)
#undef C
  }
}

}  // namespace lsa
