// lsa_api.cpp -- the C ABI of include/lsa.h: host-side validation, workspace
// sizing and kernel orchestration.  Nothing here allocates, frees or waits.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <climits>
#include <cstdint>

#include "lsa.h"
#include "lsa_internal.h"

#define LSA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline lsa_status hip_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_ERR_HIP; }

// default score-row leading dimension used by lsa_forward
inline int64_t score_ld(int32_t L) { return ((int64_t)L + 63) / 64 * 64; }

// keys per workgroup span of the flat indexer
inline int flat_span(int32_t L_max, bool direct) {
  if (direct) return lsa::DIRECT_SPAN;  // the LDS score buffer of the direct kernel
  return L_max > 65536 ? 8192 : 4096;
}

// automatic split count of the sparse attention.  Rows enough to give every CU a
// workgroup (256 and up) are not split: each wave pipelines its tiles.  Fewer rows
// are cut into splits of at most 8 32-key tiles -- one tile per wave in the one-tile
// form, two such workgroups per CU -- and into at least 256 units, so every CU holds
// a workgroup.
inline int attn_split_auto(long long rows, int32_t k_top) {
  constexpr long long kUnits = 256;
  const long long n_tiles = (k_top + 31) / 32;
  if (rows >= kUnits) return 1;
  const long long s = std::max((n_tiles + 7) / 8, (kUnits + rows - 1) / std::max<long long>(rows, 1));
  return (int)std::max<long long>(1, std::min<long long>(s, std::min<long long>(n_tiles, 64)));
}

lsa_status check_index_args(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w, const int32_t* q_pos,
                            const int32_t* kept, int32_t block_size, int32_t n_keep, int32_t B, int32_t n_q,
                            int32_t L_max, int32_t H_I, int32_t d_I, const int32_t* scores, int64_t ld) {
  if (B < 0 || n_q < 0 || L_max < 0 || H_I < 0) return LSA_ERR_INVALID_ARG;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!q_idx || !k_idx || !w || !q_pos || !scores) return LSA_ERR_INVALID_ARG;
  if (L_max < 1) return LSA_ERR_INVALID_ARG;
  if (d_I != 64 && d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (H_I < 1 || H_I > 64) return LSA_ERR_UNSUPPORTED;
  if (kept) {
    if (block_size < 1 || n_keep < 1) return LSA_ERR_INVALID_ARG;
    if (n_keep > 256 || block_size > 65536) return LSA_ERR_UNSUPPORTED;
    if (ld < (int64_t)n_keep * block_size) return LSA_ERR_INVALID_ARG;
  } else {
    if (ld < L_max) return LSA_ERR_INVALID_ARG;
  }
  return LSA_OK;
}

}  // namespace

LSA_API const char* lsa_status_string(lsa_status s) {
  switch (s) {
    case LSA_OK: return "LSA_OK";
    case LSA_ERR_INVALID_ARG: return "LSA_ERR_INVALID_ARG: invalid argument";
    case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED: shape outside the compiled variants";
    case LSA_ERR_WORKSPACE: return "LSA_ERR_WORKSPACE: workspace too small or misaligned";
    case LSA_ERR_HIP: return "LSA_ERR_HIP: kernel launch failed";
    case LSA_ERR_INTERNAL: return "LSA_ERR_INTERNAL";
    default: return "unknown lsa_status";
  }
}

LSA_API int lsa_version(void) { return 1 * 10000 + 1 * 100 + 0; }

LSA_API lsa_status lsa_index_scores(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                                    int32_t w_per_query, const int32_t* q_pos, const int32_t* kept_blocks,
                                    int32_t block_size, int32_t n_keep, int32_t B, int32_t n_q, int32_t L_max,
                                    int32_t H_I, int32_t d_I, int32_t* scores, int64_t ld_scores,
                                    void* stream) {
  lsa_status st = check_index_args(q_idx, k_idx, w, q_pos, kept_blocks, block_size, n_keep, B, n_q, L_max,
                                   H_I, d_I, scores, ld_scores);
  if (st != LSA_OK || (long long)B * n_q == 0) return st;
  lsa::IdxArgs a{};
  a.q_idx = q_idx;
  a.k_idx = k_idx;
  a.w = w;
  a.w_per_query = w_per_query ? 1 : 0;
  a.q_pos = q_pos;
  a.kept = kept_blocks;
  a.block_size = block_size;
  a.n_keep = n_keep;
  a.B = B;
  a.n_q = n_q;
  a.L_max = L_max;
  a.H_I = H_I;
  a.d_I = d_I;
  a.scores = scores;
  a.ld = ld_scores;
  a.use_direct = n_q < 8;
  a.span = flat_span(L_max, a.use_direct);
  return hip_status(lsa::launch_index_scores(a, as_stream(stream)));
}

LSA_API lsa_status lsa_block_reps(const int8_t* k_idx, int32_t B, int32_t L_max, int32_t d_I, int32_t block_size,
                                  int32_t n_blocks, int32_t* reps, void* stream) {
  if (B < 0 || L_max < 0 || n_blocks < 0 || block_size < 1) return LSA_ERR_INVALID_ARG;
  if (d_I != 64 && d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (block_size > 128) return LSA_ERR_UNSUPPORTED;
  if ((long long)n_blocks * block_size > L_max) return LSA_ERR_INVALID_ARG;
  if ((long long)B * n_blocks == 0) return LSA_OK;
  if (!k_idx || !reps) return LSA_ERR_INVALID_ARG;
  return hip_status(lsa::launch_block_reps(k_idx, B, L_max, d_I, block_size, n_blocks, reps, as_stream(stream)));
}

static size_t prefilter_ws_bytes(int32_t B, int32_t n_q, int32_t n_blocks, int32_t d_I) {
  return align_up((size_t)B * n_blocks * 2 * d_I) + align_up((size_t)B * n_q * n_blocks * 8);
}

LSA_API lsa_status lsa_block_prefilter_workspace_size(int32_t B, int32_t n_q, int32_t n_blocks, int32_t d_I,
                                                      size_t* bytes) {
  if (!bytes || B < 0 || n_q < 0 || n_blocks < 0) return LSA_ERR_INVALID_ARG;
  *bytes = prefilter_ws_bytes(B, n_q, n_blocks, d_I);
  return LSA_OK;
}

// Thresholded keep of a prefill-shaped chunk (BlkThr): where its workspace was carved.
struct BlkThrWs {
  long long* samp = nullptr;  // sampled scores, ld_s per row
  long long ld_s = 0;
  lsa::BlkThr thr{};
  int stride = 1, row_min = 0, mode = 0;
};

// Block scores and kept blocks for rows whose limbs are already in `limbs`.
// scores_private: bscores is workspace nobody reads back, so decode-shaped rows may keep
// span candidates there instead of the score table.  tw: prefill-shaped chunks take the
// thresholded keep (sample, thresholds, listing scan, list keep, fallback tiles into the
// table, table keep of the rest).
static lsa_status run_prefilter(const int8_t* q_idx, const int8_t* limbs, const int32_t* w, int32_t w_per_query,
                                const int32_t* q_pos, int32_t B, int32_t n_q, int32_t n_blocks, int32_t H_I,
                                int32_t d_I, int32_t block_size, int32_t n_keep, int32_t* kept,
                                long long* bscores, hipStream_t s, bool scores_private = false,
                                const BlkThrWs* tw = nullptr) {
  lsa::BlkCand cand{};
  if (scores_private && !lsa::blk_cand_layout((long long)B * n_q, n_q, n_blocks, n_keep, bscores,
                                              (size_t)B * n_q * n_blocks * 8, &cand))
    cand = lsa::BlkCand{};
  lsa::BlkArgs ba{};
  ba.q_idx = q_idx;
  ba.limbs = limbs;
  ba.w = w;
  ba.w_per_query = w_per_query ? 1 : 0;
  ba.q_pos = q_pos;
  ba.B = B;
  ba.n_q = n_q;
  ba.n_blocks = n_blocks;
  ba.L_max = INT_MAX;
  ba.H_I = H_I;
  ba.d_I = d_I;
  ba.block_size = block_size;
  ba.bscores = bscores;
  ba.ld = n_blocks;
  ba.span = 512;
  ba.cand = cand;
  const long long rows = (long long)B * n_q;
  const bool thr = tw != nullptr && n_q >= 8 && cand.key == nullptr;
  if (thr) {
    // sample -> thresholds -> scan appending to the lists (table rows to the table)
    lsa::BlkArgs sm = ba;
    sm.stride = tw->stride;
    sm.bscores = tw->samp;
    sm.ld = tw->ld_s;
    if (lsa::launch_block_scores(sm, s) != hipSuccess ||
        lsa::launch_blk_thresholds(tw->samp, tw->ld_s, q_pos, B, n_q, n_blocks, block_size, n_keep, tw->stride,
                                   tw->row_min, tw->mode, tw->thr, s) != hipSuccess)
      return LSA_ERR_HIP;
    ba.mode = 1;
    ba.thr = tw->thr;
  }
  hipError_t e = lsa::launch_block_scores(ba, s);
  if (e != hipSuccess) return LSA_ERR_HIP;
  if (thr) {
    // the list rows' keep; rows whose list fell short or overflowed are scored again
    // into the table, which then serves them and the table rows
    if (lsa::launch_blk_list_keep(q_pos, B, n_q, n_blocks, block_size, n_keep, tw->thr, kept, s) != hipSuccess)
      return LSA_ERR_HIP;
    ba.mode = 2;
    if (lsa::launch_block_scores(ba, s) != hipSuccess) return LSA_ERR_HIP;
  }
  lsa::BlkSelArgs sa{};
  sa.bscores = bscores;
  sa.ld = n_blocks;
  sa.q_pos = q_pos;
  sa.B = B;
  sa.n_q = n_q;
  sa.n_blocks = n_blocks;
  sa.block_size = block_size;
  sa.n_keep = n_keep;
  sa.kept = kept;
  sa.cand = cand;
  sa.rstate = thr ? tw->thr.rstate : nullptr;
  return hip_status(lsa::launch_block_select(sa, s));
}

LSA_API lsa_status lsa_block_prefilter(const int8_t* q_idx, const int32_t* reps, const int32_t* w,
                                       int32_t w_per_query, const int32_t* q_pos, int32_t B, int32_t n_q,
                                       int32_t n_blocks, int32_t H_I, int32_t d_I, int32_t block_size,
                                       int32_t n_keep, int32_t* kept_blocks, int64_t* block_scores, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (B < 0 || n_q < 0 || n_blocks < 0 || block_size < 1 || n_keep < 1) return LSA_ERR_INVALID_ARG;
  if (d_I != 64 && d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (H_I < 1 || H_I > 64 || block_size > 128 || n_keep > 256 || n_blocks > 65536) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!q_idx || !w || !q_pos || !kept_blocks || (n_blocks > 0 && !reps)) return LSA_ERR_INVALID_ARG;
  if (ws_bytes < prefilter_ws_bytes(B, n_q, n_blocks, d_I) || (ws_bytes > 0 && !ws)) return LSA_ERR_WORKSPACE;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  int8_t* limbs = static_cast<int8_t*>(ws);
  long long* bs = block_scores ? reinterpret_cast<long long*>(block_scores)
                               : reinterpret_cast<long long*>(static_cast<char*>(ws) +
                                                              align_up((size_t)B * n_blocks * 2 * d_I));
  if (n_blocks > 0) {
    hipError_t e = lsa::launch_block_limbs(reps, B, n_blocks, d_I, limbs, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
  }
  return run_prefilter(q_idx, limbs, w, w_per_query, q_pos, B, n_q, n_blocks, H_I, d_I, block_size, n_keep,
                       kept_blocks, bs, s, block_scores == nullptr);
}

LSA_API lsa_status lsa_block_cache(const int8_t* k_idx, int32_t B, int32_t L_max, int32_t d_I, int32_t block_size,
                                   int32_t n_blocks, int32_t first_block, int32_t n_update, int8_t* block_keys,
                                   void* stream) {
  if (B < 0 || L_max < 1 || block_size < 1 || n_blocks < 0 || first_block < 0 || n_update < 0 ||
      (long long)first_block + n_update > n_blocks || ((long long)first_block + n_update) * block_size > L_max)
    return LSA_ERR_INVALID_ARG;
  if (d_I != 64 && d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (block_size > 128) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_update == 0) return LSA_OK;
  if (!k_idx || !block_keys) return LSA_ERR_INVALID_ARG;
  return hip_status(lsa::launch_block_cache(k_idx, B, L_max, d_I, block_size, n_blocks, first_block, n_update,
                                            block_keys, as_stream(stream)));
}

LSA_API lsa_status lsa_block_cache_paged(const int8_t* k_idx_pool, int64_t n_slots, const int32_t* page_table,
                                         int32_t page_size, int32_t max_pages, int32_t B, int32_t d_I,
                                         int32_t block_size, int32_t n_blocks, int32_t first_block, int32_t n_update,
                                         int8_t* block_keys, void* stream) {
  if (page_size < 64 || (page_size & (page_size - 1)) != 0 || max_pages < 1 ||
      (long long)max_pages * page_size > 0x7FFFFFFFLL || n_slots < page_size || n_slots % page_size != 0 ||
      n_slots > (1LL << 31))
    return LSA_ERR_INVALID_ARG;
  const int32_t L_max = max_pages * page_size;
  if (B < 0 || block_size < 1 || n_blocks < 0 || first_block < 0 || n_update < 0 ||
      (long long)first_block + n_update > n_blocks || ((long long)first_block + n_update) * block_size > L_max)
    return LSA_ERR_INVALID_ARG;
  if (d_I != 64 && d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (block_size > 128) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_update == 0) return LSA_OK;
  if (!k_idx_pool || !page_table || !block_keys) return LSA_ERR_INVALID_ARG;
  lsa::Pages pg{};
  pg.page_table = page_table;
  pg.page_log2 = __builtin_ctz((unsigned)page_size);
  pg.max_pages = max_pages;
  pg.n_pages = (int)(n_slots / page_size);
  return hip_status(lsa::launch_block_cache(k_idx_pool, B, L_max, d_I, block_size, n_blocks, first_block, n_update,
                                            block_keys, as_stream(stream), pg));
}

LSA_API lsa_status lsa_topk_workspace_size(int32_t B, int32_t n_q, int32_t L_max, int32_t k, size_t* bytes) {
  if (!bytes || B < 0 || n_q < 0 || L_max < 0 || k < 0) return LSA_ERR_INVALID_ARG;
  *bytes = lsa::topk_ws_bytes((long long)B * n_q, L_max);
  return LSA_OK;
}

LSA_API lsa_status lsa_topk(const int32_t* scores, int64_t ld_scores, const int32_t* q_pos,
                            const int32_t* kept_blocks, int32_t block_size, int32_t n_keep, int32_t B, int32_t n_q,
                            int32_t L_max, int32_t k, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                            void* stream) {
  if (B < 0 || n_q < 0 || L_max < 0) return LSA_ERR_INVALID_ARG;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  if (k < 1) return LSA_ERR_INVALID_ARG;
  if (k > 4096) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!scores || !q_pos || !idx || L_max < 1) return LSA_ERR_INVALID_ARG;
  if (kept_blocks) {
    if (block_size < 1 || n_keep < 1) return LSA_ERR_INVALID_ARG;
    if (n_keep > 256) return LSA_ERR_UNSUPPORTED;
    if (ld_scores < (int64_t)n_keep * block_size) return LSA_ERR_INVALID_ARG;
  } else if (ld_scores < L_max) {
    return LSA_ERR_INVALID_ARG;
  }
  lsa::TopkArgs a{};
  a.scores = scores;
  a.ld = ld_scores;
  a.q_pos = q_pos;
  a.kept = kept_blocks;
  a.block_size = block_size;
  a.n_keep = n_keep;
  a.B = B;
  a.n_q = n_q;
  a.L_max = L_max;
  a.k = k;
  a.idx = idx;
  a.count = count;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return hip_status(lsa::launch_topk(a, as_stream(stream)));
}

// split count of the sparse attention: at most one 32-key tile per split, and at most
// 64 splits (the merge keeps a weight per split and head in LDS)
static int resolve_split(int32_t B, int32_t n_q, int32_t k_top, int32_t n_split) {
  const long long rows = (long long)B * n_q;
  const int n_tiles = (k_top + 31) / 32;
  const int want = n_split <= 0 ? attn_split_auto(rows, k_top) : n_split;
  return std::max(1, std::min(std::min(want, n_tiles), 64));
}

static size_t attn_ws_bytes(long long rows, int32_t H_q, int32_t d, int split) {
  if (split <= 1) return 0;
  const long long units = rows * split;
  return align_up((size_t)units * H_q * d * 4) + align_up((size_t)units * H_q * 4);
}

LSA_API lsa_status lsa_sparse_attn_workspace_size(int32_t B, int32_t n_q, int32_t H_q, int32_t d, int32_t k,
                                                  int32_t n_split, size_t* bytes) {
  if (!bytes || B < 0 || n_q < 0 || H_q < 0 || d < 0 || k < 1) return LSA_ERR_INVALID_ARG;
  const int split = resolve_split(B, n_q, k, n_split);
  *bytes = attn_ws_bytes((long long)B * n_q, H_q, d, split);
  return LSA_OK;
}

static lsa_status run_attn(const void* q, const void* k, const void* v, const int32_t* idx, int32_t B, int32_t n_q,
                           int32_t L_max, int32_t H_q, int32_t d, int32_t k_top, float scale, int split, void* out,
                           float* lse, void* ws, hipStream_t s, long long kv_pool = 0) {
  lsa::AttnArgs a{};
  a.kv_pool = kv_pool;
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.B = B;
  a.n_q = n_q;
  a.L_max = L_max;
  a.H_q = H_q;
  a.d = d;
  a.k_top = k_top;
  a.scale = scale;
  a.n_split = split;
  a.out = out;
  a.lse = lse;
  a.ws = static_cast<float*>(ws);
  return hip_status(lsa::launch_sparse_attn(a, s));
}

LSA_API lsa_status lsa_sparse_attn(const void* q, const void* k, const void* v, const int32_t* idx, int32_t B,
                                   int32_t n_q, int32_t L_max, int32_t H_q, int32_t d, int32_t k_top, float scale,
                                   int32_t n_split, void* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (B < 0 || n_q < 0 || L_max < 0 || k_top < 1 || H_q < 1) return LSA_ERR_INVALID_ARG;
  if (d != 128) return LSA_ERR_UNSUPPORTED;
  if (H_q > 16 || k_top > 65536) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!q || !k || !v || !idx || !out || L_max < 1) return LSA_ERR_INVALID_ARG;
  const int split = resolve_split(B, n_q, k_top, n_split);
  const size_t need = attn_ws_bytes((long long)B * n_q, H_q, d, split);
  if (ws_bytes < need || (need > 0 && !ws)) return LSA_ERR_WORKSPACE;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  return run_attn(q, k, v, idx, B, n_q, L_max, H_q, d, k_top, scale, split, out, lse, ws, as_stream(stream));
}

LSA_API lsa_status lsa_sparse_attn_pool(const void* q, const void* k_pool, const void* v_pool, const int32_t* idx,
                                        int32_t B, int32_t n_q, int64_t n_slots, int32_t H_q, int32_t d,
                                        int32_t k_top, float scale, int32_t n_split, void* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (B < 0 || n_q < 0 || n_slots < 0 || n_slots > (1LL << 31) || k_top < 1 || H_q < 1) return LSA_ERR_INVALID_ARG;
  if (d != 128) return LSA_ERR_UNSUPPORTED;
  if (H_q > 16 || k_top > 65536) return LSA_ERR_UNSUPPORTED;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!q || !k_pool || !v_pool || !idx || !out || n_slots < 1) return LSA_ERR_INVALID_ARG;
  const int split = resolve_split(B, n_q, k_top, n_split);
  const size_t need = attn_ws_bytes((long long)B * n_q, H_q, d, split);
  if (ws_bytes < need || (need > 0 && !ws)) return LSA_ERR_WORKSPACE;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  const int32_t L_clip = n_slots > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int32_t)n_slots;
  return run_attn(q, k_pool, v_pool, idx, B, n_q, L_clip, H_q, d, k_top, scale, split, out, lse, ws,
                  as_stream(stream), n_slots);
}

// ------------------------------------------------------------------------------------------ forward
namespace {

struct FwdPlan {
  bool decode_like;     // n_q == 1: chunks are groups of sequences
  long long per_row;    // workspace bytes per chunk row
  size_t fixed;         // workspace bytes independent of the chunk
  int64_t ld;           // score row stride
  int32_t n_blocks;
  size_t il_bytes;      // the token stage's interleaved key copy (part of fixed), 0 = none
};

lsa_status check_forward(const lsa_forward_args* a) {
  if (!a) return LSA_ERR_INVALID_ARG;
  if (a->mode != LSA_MODE_PREFILL && a->mode != LSA_MODE_DECODE) return LSA_ERR_INVALID_ARG;
  if (a->B < 0 || a->n_q < 0 || a->L_max < 1 || a->k_top < 1) return LSA_ERR_INVALID_ARG;
  if (a->mode == LSA_MODE_DECODE && a->n_q != 1) return LSA_ERR_INVALID_ARG;
  if (a->d_I != 64 && a->d_I != 128) return LSA_ERR_UNSUPPORTED;
  if (a->H_I < 1 || a->H_I > 64 || a->d != 128 || a->H_q < 1 || a->H_q > 16) return LSA_ERR_UNSUPPORTED;
  if (a->k_top > 4096) return LSA_ERR_UNSUPPORTED;
  if (a->select_mode < LSA_SELECT_AUTO || a->select_mode > LSA_SELECT_FORCE_OVERFLOW) return LSA_ERR_INVALID_ARG;
  if (a->two_stage < 0 || a->two_stage > 2) return LSA_ERR_INVALID_ARG;
  if (a->two_stage) {
    if (a->block_size < 1 || a->n_keep < 1) return LSA_ERR_INVALID_ARG;
    if (a->block_size > 128 || a->L_max / a->block_size > 65536) return LSA_ERR_UNSUPPORTED;
    if (a->two_stage == 1 && a->n_keep > 256) return LSA_ERR_UNSUPPORTED;  // the token stage's kept table
    // pooled blocks: the list is the keys of the kept blocks
    if (a->two_stage == 2 && (long long)a->n_keep * a->block_size != a->k_top) return LSA_ERR_INVALID_ARG;
  } else if (a->block_keys) {
    return LSA_ERR_INVALID_ARG;
  }
  if (a->page_table) {
    if (a->page_size < 64 || (a->page_size & (a->page_size - 1)) != 0 || a->max_pages < 1 ||
        (long long)a->max_pages * a->page_size != a->L_max || a->n_slots < a->page_size ||
        a->n_slots % a->page_size != 0 || a->n_slots > (1ll << 31))
      return LSA_ERR_INVALID_ARG;
    // block modes over paged caches: the token stage's scores and top-k in one kernel
    if (a->two_stage == 1 && !(a->n_keep <= 256 && (long long)a->n_keep * a->block_size <= lsa::KSEL_SLOTS))
      return LSA_ERR_UNSUPPORTED;
  }
  if ((long long)a->B * a->n_q == 0) return LSA_OK;
  if (!a->q_idx || !a->k_idx || !a->w || !a->q_pos || !a->q || !a->k || !a->v || !a->idx || !a->out)
    return LSA_ERR_INVALID_ARG;
  return LSA_OK;
}

// pages of the chunk whose first sequence is b0 (page_table == nullptr: contiguous caches)
lsa::Pages chunk_pages(const lsa_forward_args* a, int32_t b0) {
  lsa::Pages pg{};
  if (!a->page_table) return pg;
  pg.page_table = a->page_table + (long long)b0 * a->max_pages;
  pg.page_log2 = __builtin_ctz((unsigned)a->page_size);
  pg.max_pages = a->max_pages;
  pg.n_pages = (int)(a->n_slots / a->page_size);
  return pg;
}

// Thresholded selection (the score table only for short rows and fallbacks) applies to
// flat chunks of at least 8 queries per sequence whose rows may exceed thr_cap(k) keys.
bool thr_applies(const lsa_forward_args* a) {
  return !a->two_stage && a->select_mode != LSA_SELECT_TABLE && a->n_q >= 8 && a->k_top <= lsa::THR_MAX_K &&
         a->L_max <= lsa::THR_MAX_L && a->L_max > lsa::thr_row_min(a->k_top);
}
// sampled scores per row (leading dimension)
int64_t thr_ld(int32_t L_max, int32_t k) {
  const int st = lsa::thr_stride(k);
  return ((int64_t)(L_max - 1) / st + 1 + 63) / 64 * 64;
}
// its workspace for a chunk of `rows` rows: sampled scores, threshold, state and count
// per row, and the candidate lists (slots, scores)
size_t thr_ws_bytes(const lsa_forward_args* a, long long rows) {
  if (!thr_applies(a)) return 0;
  const size_t cap = (size_t)lsa::thr_cap(a->k_top);
  return align_up((size_t)rows * thr_ld(a->L_max, a->k_top) * 4) + 3 * align_up((size_t)rows * 4) +
         2 * align_up((size_t)rows * cap * 4);
}

// Thresholded block keep (block modes, prefill-shaped chunks): rows of more than
// blk_thr_row_min(n_keep) blocks, where the sample costs at most 1/BLK_THR_MIN_STRIDE
// of the scan and fits the threshold kernel.
bool blk_thr_applies(const lsa_forward_args* a) {
  if (!a->two_stage || a->select_mode == LSA_SELECT_TABLE || a->n_q < 8 || a->n_keep < 2 || a->n_keep > 2048)
    return false;
  const int nb = a->L_max / a->block_size, st = lsa::blk_thr_stride(a->n_keep);
  return st >= lsa::BLK_THR_MIN_STRIDE && nb > lsa::blk_thr_row_min(a->n_keep) && nb <= lsa::BLK_THR_MAX_B &&
         (nb + st - 1) / st <= lsa::BLK_THR_MAX_SAMPLES;
}
// sampled scores per row (leading dimension, a multiple of 8: 64-byte rows)
int64_t blk_thr_ld(const lsa_forward_args* a) {
  const int st = lsa::blk_thr_stride(a->n_keep);
  return ((int64_t)(a->L_max / a->block_size + st - 1) / st + 7) / 8 * 8;
}
// its workspace for a chunk of `rows` rows: samples, threshold, state, count, lists, and
// the fallback tile marks, list and count (a tile per row at most)
size_t blk_thr_ws_bytes(const lsa_forward_args* a, long long rows) {
  if (!blk_thr_applies(a)) return 0;
  const size_t cap = (size_t)lsa::blk_thr_cap(a->n_keep);
  return align_up((size_t)rows * blk_thr_ld(a) * 8) + align_up((size_t)rows * 8) + 2 * align_up((size_t)rows * 4) +
         align_up((size_t)rows * cap * 4) + align_up((size_t)rows * cap * 8) + 2 * align_up((size_t)rows * 4) +
         align_up(4);
}

// Two-stage rows whose kept slots fit one workgroup's LDS: the token stage and its top-k
// run as one kernel, with no token score table.
bool kept_fused(const lsa_forward_args* a) {
  return a->two_stage == 1 && a->n_keep <= 256 && (long long)a->n_keep * a->block_size <= lsa::KSEL_SLOTS;
}

// The one-kernel token stage reads its keys from a chunk-interleaved copy, built at the
// start of the call, where the copy pays: block sizes a multiple of 64 and at least 8
// kept-key reads per cached key (many queries per sequence: prefill).
bool kept_il(const lsa_forward_args* a) {
  if (!kept_fused(a) || a->block_size % 64 != 0) return false;
  const double reads = (double)a->B * a->n_q * a->n_keep * a->block_size;
  return reads >= 8.0 * (double)a->B * a->L_max;
}

// with_il = false: the plan without the interleaved copy (a workspace too small for it)
FwdPlan plan_forward(const lsa_forward_args* a, bool with_il = true) {
  FwdPlan p{};
  p.decode_like = a->n_q == 1;
  if (a->two_stage) {
    p.n_blocks = a->L_max / a->block_size;
    // the token stage's score rows (pooled blocks have none)
    p.ld = (a->two_stage == 2 || kept_fused(a)) ? 0 : (int64_t)a->n_keep * a->block_size;
    p.per_row = p.ld * 4 + (long long)p.n_blocks * 8 + (a->kept_blocks ? 0 : (long long)a->n_keep * 4) + 64;
    if (blk_thr_applies(a)) p.per_row += blk_thr_ld(a) * 8 + 24 + (long long)lsa::blk_thr_cap(a->n_keep) * 12;
    // the block-key cache, unless the caller keeps one
    p.fixed = a->block_keys ? 0 : align_up((size_t)a->B * p.n_blocks * 2 * a->d_I);
    p.il_bytes = with_il && kept_il(a) ? align_up(lsa::kidx_interleave_bytes(a->B, a->L_max, a->d_I)) : 0;
    p.fixed += p.il_bytes;
  } else {
    p.n_blocks = 0;
    p.ld = score_ld(a->L_max);
    p.per_row = p.ld * 4;
    if (thr_applies(a)) p.per_row += thr_ld(a->L_max, a->k_top) * 4 + 2LL * lsa::thr_cap(a->k_top) * 4 + 12;
    p.fixed = 0;
  }
  return p;
}

// top-k workspace of chunks of `rows` rows: the split top-k's, and the decode
// selection's state for every chunk of fewer than 8 queries per sequence that occurs
// (all chunks when n_q == 1; a chunk of fewer rows needs no more)
size_t topk_ws_for(const lsa_forward_args* a, long long rows) {
  long long dec_rows = 0;
  if (a->n_q == 1 || rows < 8) dec_rows = rows;
  else if (a->n_q % rows > 0 && a->n_q % rows < 8) dec_rows = a->n_q % rows;  // the last, short chunk
  const size_t dec = dec_rows > 0 ? lsa::dec_sel_ws_bytes(dec_rows, a->L_max, a->k_top) : 0;
  return std::max(dec, lsa::topk_ws_bytes(rows, a->L_max));
}

// workspace for a chunk of `rows` rows
size_t chunk_bytes(const lsa_forward_args* a, const FwdPlan& p, long long rows) {
  size_t s = p.fixed;
  s += align_up((size_t)rows * p.ld * 4);                                   // scores
  if (a->two_stage) {
    s += align_up((size_t)rows * p.n_blocks * 8);                           // block scores
    if (!a->kept_blocks) s += align_up((size_t)rows * a->n_keep * 4);       // kept lists
  }
  const int split = resolve_split(1, (int32_t)rows, a->k_top, a->attn_split);
  s += attn_ws_bytes(rows, a->H_q, a->d, split);
  if (!a->two_stage) s += align_up(topk_ws_for(a, rows));
  s += thr_ws_bytes(a, rows);
  s += blk_thr_ws_bytes(a, rows);
  return s;
}

long long total_rows(const lsa_forward_args* a) { return a->n_q == 1 ? (long long)a->B : (long long)a->n_q; }

constexpr long long kChunkBudget = 8ll << 30;  // default chunk budget (bytes)

// rows per chunk for a workspace of ws_bytes (0 if even one row does not fit)
long long plan_rows(const lsa_forward_args* a, const FwdPlan& p, size_t ws_bytes);

// the plan and rows per chunk for a workspace of ws_bytes: with the interleaved key copy
// where it fits, else without it (rows 0: not even one row fits)
FwdPlan plan_for(const lsa_forward_args* a, size_t ws_bytes, long long* rows) {
  FwdPlan p = plan_forward(a);
  *rows = plan_rows(a, p, ws_bytes);
  if (*rows == 0 && p.il_bytes > 0) {
    p = plan_forward(a, false);
    *rows = plan_rows(a, p, ws_bytes);
  }
  return p;
}

// Chunks of equal size for n_rows rows in chunks of at most fit rows: as many chunks as
// fit requires, none of them a short tail (a tail of a few rows would run the
// decode-shaped kernels and pay every stage's launches for little work).
long long balanced_rows(long long n_rows, long long fit) {
  const long long n_chunks = (n_rows + fit - 1) / fit;
  return (n_rows + n_chunks - 1) / n_chunks;
}

long long plan_rows(const lsa_forward_args* a, const FwdPlan& p, size_t ws_bytes) {
  const long long n_rows = total_rows(a);
  long long rows = a->chunk_rows > 0 ? std::min<long long>(a->chunk_rows, n_rows) : n_rows;
  if (chunk_bytes(a, p, rows) <= ws_bytes) return rows;
  if (a->chunk_rows > 0 || chunk_bytes(a, p, 1) > ws_bytes) return 0;
  long long lo = 1, hi = rows;
  while (lo < hi) {
    const long long mid = (lo + hi + 1) / 2;
    if (chunk_bytes(a, p, mid) <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  return balanced_rows(n_rows, lo);
}

}  // namespace

namespace {

// A chunk of flat rows of few queries per sequence takes the decode selection: the
// indexer builds each row's histogram and span candidate lists, and the top-k
// finishes every row from them (no score table in between) -- where its state fits
// the chunk's top-k workspace of topk_ws_size bytes.
bool chunk_fused(const lsa_forward_args* a, int32_t nb, int32_t ni, size_t topk_ws_size) {
  const size_t need = lsa::dec_sel_ws_bytes((long long)nb * ni, a->L_max, a->k_top);
  return !a->two_stage && ni < 8 && need > 0 && need <= topk_ws_size;
}

bool chunk_thr(const lsa_forward_args* a, int32_t nb, int32_t ni, size_t topk_ws_size) {
  return thr_applies(a) && !chunk_fused(a, nb, ni, topk_ws_size);
}

// chunks of lsa_forward for `rows` rows per chunk, as (b0, nb, i0, ni)
template <typename F>
void for_each_chunk(const lsa_forward_args* a, long long rows, F f) {
  if (a->n_q == 1) {
    for (long long b0 = 0; b0 < a->B; b0 += rows) f((int32_t)b0, (int32_t)std::min<long long>(rows, a->B - b0), 0, 1);
  } else {
    for (int32_t b = 0; b < a->B; ++b)
      for (long long i0 = 0; i0 < a->n_q; i0 += rows)
        f(b, 1, (int32_t)i0, (int32_t)std::min<long long>(rows, a->n_q - i0));
  }
}

// stage codes of lsa_forward in launch order (rows per chunk already planned)
std::vector<int32_t> forward_stages(const lsa_forward_args* a, const FwdPlan& p, long long rows) {
  std::vector<int32_t> st;
  if (a->two_stage && ((p.n_blocks > 0 && !a->block_keys) || p.il_bytes > 0)) st.push_back(LSA_STAGE_BLOCK_REPS);
  const size_t topk_ws_size = a->two_stage ? 0 : topk_ws_for(a, rows);
  for_each_chunk(a, rows, [&](int32_t, int32_t nb, int32_t, int32_t ni) {
    if (a->two_stage) st.push_back(LSA_STAGE_BLOCK_PREFILTER);
    if (a->two_stage == 2 || kept_fused(a)) {
      st.push_back(a->two_stage == 2 ? LSA_STAGE_EXPAND : LSA_STAGE_INDEX_SELECT);
      st.push_back(LSA_STAGE_SPARSE_ATTN);
      return;
    }
    const bool thr = chunk_thr(a, nb, ni, topk_ws_size);
    if (thr) st.push_back(LSA_STAGE_SAMPLE);
    st.push_back(chunk_fused(a, nb, ni, topk_ws_size) || thr ? LSA_STAGE_INDEX_SELECT : LSA_STAGE_INDEX_SCORES);
    st.push_back(LSA_STAGE_TOPK);
    st.push_back(LSA_STAGE_SPARSE_ATTN);
  });
  return st;
}

}  // namespace

LSA_API lsa_status lsa_forward_workspace_size(const lsa_forward_args* a, size_t* bytes) {
  if (!bytes) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_forward(a);
  if (st != LSA_OK) return st;
  if ((long long)a->B * a->n_q == 0) {
    *bytes = 0;
    return LSA_OK;
  }
  const FwdPlan p = plan_forward(a);
  const long long n_rows = total_rows(a);
  long long rows = a->chunk_rows > 0 ? std::min<long long>(a->chunk_rows, n_rows)
                                     : balanced_rows(n_rows, std::max<long long>(1, kChunkBudget / p.per_row));
  *bytes = chunk_bytes(a, p, rows);
  return LSA_OK;
}

LSA_API lsa_status lsa_forward(const lsa_forward_args* a, void* ws, size_t ws_bytes, void* stream) {
  lsa_status st = check_forward(a);
  if (st != LSA_OK) return st;
  if ((long long)a->B * a->n_q == 0) return LSA_OK;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const long long n_rows = total_rows(a);

  // rows per chunk: requested, else the most that fit
  long long rows = 0;
  const FwdPlan p = plan_for(a, ws_bytes, &rows);
  if (rows == 0 || (!ws && chunk_bytes(a, p, rows) > 0)) return LSA_ERR_WORKSPACE;
  (void)n_rows;
  if (a->stage_events != nullptr &&
      (long long)a->n_stage_events < 1 + (long long)forward_stages(a, p, rows).size())
    return LSA_ERR_INVALID_ARG;
  if (a->page_table && !a->two_stage) {
    // paged caches: flat chunks of fewer than 8 queries per sequence must take the decode selection
    const size_t tws = topk_ws_for(a, rows);
    bool ok = true;
    for_each_chunk(a, rows, [&](int32_t, int32_t nb, int32_t, int32_t ni) {
      ok = ok && (ni >= 8 || chunk_fused(a, nb, ni, tws));
    });
    if (!ok) return LSA_ERR_WORKSPACE;
  }
  int32_t n_marked = 0;
  // records the next stage event (if the caller asked for them)
  auto mark = [&]() -> bool {
    if (a->stage_events == nullptr) return true;
    return hipEventRecord(static_cast<hipEvent_t>(a->stage_events[n_marked++]), s) == hipSuccess;
  };
  if (!mark()) return LSA_ERR_HIP;

  // workspace carve-up
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  const int8_t* limbs = a->block_keys;  // block-key cache: the caller's, else built here
  int8_t* limbs_ws = nullptr;
  if (a->two_stage && !a->block_keys) {
    limbs_ws = reinterpret_cast<int8_t*>(base + off);
    limbs = limbs_ws;
    off += align_up((size_t)a->B * p.n_blocks * 2 * a->d_I);
  }
  int8_t* k_il = nullptr;  // the token stage's interleaved keys
  if (p.il_bytes > 0) {
    k_il = reinterpret_cast<int8_t*>(base + off);
    off += p.il_bytes;
  }
  int32_t* sc = reinterpret_cast<int32_t*>(base + off);
  off += align_up((size_t)rows * p.ld * 4);
  long long* bsc = nullptr;
  int32_t* kept_ws = nullptr;
  if (a->two_stage) {
    bsc = reinterpret_cast<long long*>(base + off);
    off += align_up((size_t)rows * p.n_blocks * 8);
    if (!a->kept_blocks) {
      kept_ws = reinterpret_cast<int32_t*>(base + off);
      off += align_up((size_t)rows * a->n_keep * 4);
    }
  }
  void* attn_ws = base + off;
  off += attn_ws_bytes(rows, a->H_q, a->d, resolve_split(1, (int32_t)rows, a->k_top, a->attn_split));
  void* topk_ws = a->two_stage ? nullptr : static_cast<void*>(base + off);
  const size_t topk_ws_size = a->two_stage ? 0 : topk_ws_for(a, rows);
  if (!a->two_stage) off += align_up(topk_ws_size);
  // thresholded selection: sampled scores, per-row threshold / state / count, candidate lists
  int32_t* thr_samp = nullptr;
  lsa::ThrArgs thr{};
  const int64_t ld_s = thr_ld(a->L_max, a->k_top);
  if (thr_applies(a)) {
    thr.cap = lsa::thr_cap(a->k_top);
    thr.row_min = lsa::thr_row_min(a->k_top);
    thr_samp = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * ld_s * 4);
    thr.theta = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    thr.rstate = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    thr.cnt = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    thr.lslot = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * thr.cap * 4);
    thr.lscore = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * thr.cap * 4);
  }
  // thresholded block keep: sampled block scores, per-row threshold / state / count, lists
  BlkThrWs bt;
  const bool use_bt = blk_thr_applies(a);
  if (use_bt) {
    bt.stride = lsa::blk_thr_stride(a->n_keep);
    bt.row_min = lsa::blk_thr_row_min(a->n_keep);
    bt.mode = a->select_mode == LSA_SELECT_FORCE_SHORT ? 1 : a->select_mode == LSA_SELECT_FORCE_OVERFLOW ? 2 : 0;
    bt.ld_s = blk_thr_ld(a);
    bt.thr.cap = lsa::blk_thr_cap(a->n_keep);
    bt.samp = reinterpret_cast<long long*>(base + off);
    off += align_up((size_t)rows * bt.ld_s * 8);
    bt.thr.theta = reinterpret_cast<long long*>(base + off);
    off += align_up((size_t)rows * 8);
    bt.thr.rstate = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    bt.thr.cnt = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    bt.thr.lblk = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * bt.thr.cap * 4);
    bt.thr.lscore = reinterpret_cast<long long*>(base + off);
    off += align_up((size_t)rows * bt.thr.cap * 8);
    bt.thr.tflag = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    bt.thr.tlist = reinterpret_cast<int32_t*>(base + off);
    off += align_up((size_t)rows * 4);
    bt.thr.tcnt = reinterpret_cast<int32_t*>(base + off);
    off += align_up(4);
  }

  const int32_t d_I = a->d_I, H_I = a->H_I, H_q = a->H_q, d = a->d, L = a->L_max, kt = a->k_top;
  // one split count for every chunk, so no chunk needs more attention workspace than sized
  const int split = resolve_split(1, (int32_t)rows, kt, a->attn_split);
  // caches derived from the keys, one stage: the block-key cache and the interleaved keys
  const bool build_limbs = a->two_stage && p.n_blocks > 0 && limbs_ws;
  if (build_limbs && lsa::launch_block_cache(a->k_idx, a->B, L, d_I, a->block_size, p.n_blocks, 0, p.n_blocks,
                                             limbs_ws, s, chunk_pages(a, 0)) != hipSuccess)
    return LSA_ERR_HIP;
  if (k_il && lsa::launch_kidx_interleave(a->k_idx, a->B, L, d_I, chunk_pages(a, 0), k_il, s) != hipSuccess)
    return LSA_ERR_HIP;
  if ((build_limbs || k_il) && !mark()) return LSA_ERR_HIP;

  // one chunk: sequences [b0, b0+nb) x queries [i0, i0+ni) (either nb == 1 or ni == n_q == 1)
  auto run_chunk = [&](int32_t b0, int32_t nb, int32_t i0, int32_t ni) -> lsa_status {
    const long long r0 = (long long)b0 * a->n_q + i0;  // first flattened row
    const int8_t* qi = a->q_idx + r0 * H_I * d_I;
    const bool paged = a->page_table != nullptr;  // caches are pools: no per-sequence offset
    const int8_t* ki = a->k_idx + (paged ? 0ll : (long long)b0 * L * d_I);
    const int32_t* wq = a->w_per_query ? a->w + r0 * H_I : a->w;
    const int32_t* qp = a->q_pos + r0;
    const char* qq = static_cast<const char*>(a->q) + r0 * H_q * d * 2;
    const char* kk = static_cast<const char*>(a->k) + (paged ? 0ll : (long long)b0 * L * d * 2);
    const char* vv = static_cast<const char*>(a->v) + (paged ? 0ll : (long long)b0 * L * d * 2);
    int32_t* ix = a->idx + r0 * kt;
    int32_t* cnt = a->count ? a->count + r0 : nullptr;
    char* oo = static_cast<char*>(a->out) + r0 * H_q * d * 2;
    float* ls = a->lse ? a->lse + r0 * H_q : nullptr;
    const int32_t* kept = nullptr;
    lsa::IdxArgs ia{};
    ia.q_idx = qi;
    ia.k_idx = ki;
    ia.w = wq;
    ia.w_per_query = a->w_per_query ? 1 : 0;
    ia.q_pos = qp;
    ia.B = nb;
    ia.n_q = ni;
    ia.L_max = L;
    ia.H_I = H_I;
    ia.d_I = d_I;
    ia.scores = sc;
    ia.ld = p.ld;
    ia.pages = chunk_pages(a, b0);
    if (a->two_stage) {
      int32_t* kout = a->kept_blocks ? a->kept_blocks + r0 * a->n_keep : kept_ws;
      lsa_status st2 = run_prefilter(qi, limbs + (long long)b0 * p.n_blocks * 2 * d_I, wq, a->w_per_query, qp, nb,
                                     ni, p.n_blocks, H_I, d_I, a->block_size, a->n_keep, kout, bsc, s, true,
                                     use_bt ? &bt : nullptr);
      if (st2 != LSA_OK) return st2;
      kept = kout;
      ia.kept = kept;
      ia.block_size = a->block_size;
      ia.n_keep = a->n_keep;
      if (!mark()) return LSA_ERR_HIP;
      if (a->two_stage == 2 || kept_fused(a)) {
        hipError_t e;
        if (a->two_stage == 2) {
          // pooled blocks: the list is every key of the kept blocks the query may see
          e = lsa::launch_expand(kept, qp, (long long)nb * ni, a->block_size, a->n_keep, kt, ix, cnt, s,
                                 chunk_pages(a, b0), ni);
        } else {
          // the token stage and its top-k in one kernel
          ia.k_il = k_il ? k_il + (long long)b0 * ((L + 63) / 64) * 64 * d_I : nullptr;
          e = lsa::launch_kept_select(ia, kt, ix, cnt, s);
        }
        if (e != hipSuccess || !mark()) return LSA_ERR_HIP;
        lsa_status sa = run_attn(qq, kk, vv, ix, nb, ni, L, H_q, d, kt, a->scale, split, oo, ls, attn_ws, s,
                                 paged ? (long long)a->n_slots : 0ll);
        if (sa != LSA_OK) return sa;
        return mark() ? LSA_OK : LSA_ERR_HIP;
      }
    }
    ia.use_direct = a->two_stage ? true : ni < 8;
    ia.span = flat_span(L, ia.use_direct);
    lsa::TopkArgs ta{};
    ta.scores = sc;
    ta.ld = p.ld;
    ta.q_pos = qp;
    ta.kept = kept;
    ta.block_size = a->block_size;
    ta.n_keep = a->n_keep;
    ta.B = nb;
    ta.n_q = ni;
    ta.pages = ia.pages;  // paged caches: the top-k writes pool rows
    ta.L_max = L;
    ta.k = kt;
    ta.idx = ix;
    ta.count = cnt;
    ta.ws = topk_ws;
    ta.ws_bytes = topk_ws_size;
    if (chunk_fused(a, nb, ni, topk_ws_size)) {
      // the indexer builds each row's selection state (histogram, span candidate lists)
      lsa::DecLayout dl;
      if (!lsa::dec_sel_layout((long long)nb * ni, L, kt, &dl)) return LSA_ERR_INTERNAL;
      ta.hist_ready = true;
      ia.sel_base = static_cast<int*>(topk_ws);
      ia.sel_rec_ints = dl.rec_ints;
      ia.sel_parts = dl.parts;
      ia.sel_lcap = dl.lcap;
      ia.k_top = kt;
    }
    if (chunk_thr(a, nb, ni, topk_ws_size)) {
      // Thresholded selection: score a sample of every row's keys and set its
      // threshold (short rows keep the table) ...
      const long long rows_c = (long long)nb * ni;
      const int mode = a->select_mode == LSA_SELECT_FORCE_SHORT ? 1 : a->select_mode == LSA_SELECT_FORCE_OVERFLOW ? 2 : 0;
      lsa::IdxArgs sa = ia;
      sa.stride = lsa::thr_stride(kt);
      sa.row_min = thr.row_min;  // table rows need no threshold
      sa.scores = thr_samp;
      sa.ld = ld_s;
      if (lsa::launch_index_scores(sa, s) != hipSuccess) return LSA_ERR_HIP;
      if (lsa::launch_thresholds(thr_samp, ld_s, qp, rows_c, L, kt, sa.stride, mode, thr, s) != hipSuccess ||
          !mark())
        return LSA_ERR_HIP;
      // ... the scan appends each list row's candidates (table rows store their scores) ...
      ia.thr = thr;
      if (lsa::launch_index_scores(ia, s) != hipSuccess || !mark()) return LSA_ERR_HIP;
      // ... the list rows' top-k from their lists; rows whose list fell short or
      // overflowed are scored again into the table, and the top-k of the table rows
      if (lsa::launch_list_topk(qp, rows_c, L, kt, thr, ix, cnt, ni, ia.pages, s) != hipSuccess) return LSA_ERR_HIP;
      lsa::IdxArgs fa = ia;
      fa.thr = lsa::ThrArgs{};
      fa.tile_filter = thr.rstate;
      if (lsa::launch_index_scores(fa, s) != hipSuccess) return LSA_ERR_HIP;
      ta.row_state = thr.rstate;
      if (lsa::launch_topk(ta, s) != hipSuccess || !mark()) return LSA_ERR_HIP;
    } else {
      if (lsa::launch_index_scores(ia, s) != hipSuccess || !mark()) return LSA_ERR_HIP;
      if (lsa::launch_topk(ta, s) != hipSuccess || !mark()) return LSA_ERR_HIP;
    }
    lsa_status sa = run_attn(qq, kk, vv, ix, nb, ni, L, H_q, d, kt, a->scale, split, oo, ls, attn_ws, s,
                             paged ? (long long)a->n_slots : 0ll);
    if (sa != LSA_OK) return sa;
    return mark() ? LSA_OK : LSA_ERR_HIP;
  };

  lsa_status result = LSA_OK;
  for_each_chunk(a, rows, [&](int32_t b0, int32_t nb, int32_t i0, int32_t ni) {
    if (result == LSA_OK) result = run_chunk(b0, nb, i0, ni);
  });
  return result;
}

LSA_API lsa_status lsa_forward_stages(const lsa_forward_args* a, size_t ws_bytes, int32_t* codes, int32_t max_codes,
                                      int32_t* n_stages) {
  if (!n_stages || max_codes < 0) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_forward(a);
  if (st != LSA_OK) return st;
  *n_stages = 0;
  if ((long long)a->B * a->n_q == 0) return LSA_OK;
  long long rows = 0;
  const FwdPlan p = plan_for(a, ws_bytes, &rows);
  if (rows == 0) return LSA_ERR_WORKSPACE;
  const std::vector<int32_t> v = forward_stages(a, p, rows);
  for (size_t i = 0; codes != nullptr && i < v.size() && (long long)i < max_codes; ++i) codes[i] = v[i];
  *n_stages = (int32_t)v.size();
  return LSA_OK;
}

LSA_API lsa_status lsa_forward_plan(const lsa_forward_args* a, size_t ws_bytes, int64_t* chunk_rows,
                                    int32_t* attn_split) {
  if (!chunk_rows || !attn_split) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_forward(a);
  if (st != LSA_OK) return st;
  if ((long long)a->B * a->n_q == 0) {
    *chunk_rows = 0;
    *attn_split = 1;
    return LSA_OK;
  }
  long long rows = 0;
  (void)plan_for(a, ws_bytes, &rows);
  if (rows == 0) return LSA_ERR_WORKSPACE;
  *chunk_rows = rows;
  *attn_split = resolve_split(1, (int32_t)rows, a->k_top, a->attn_split);
  return LSA_OK;
}


// ---------------------------------------------------------------------------------
// flat semantic search

static lsa_status check_sem_params(const lsa_semantic_params* prm, int d_idx, lsa::SemParams* sp) {
  if (!prm) return LSA_ERR_INVALID_ARG;
  const lsa_semantic_params& p = *prm;
  if (p.n_cluster < 1 || p.n_pool < 1 || p.n_bavg < 1 || p.n_bmax < 1 || p.n_cluster % p.n_pool != 0 ||
      p.n_cluster % p.n_bavg != 0 || p.n_bmax % p.n_pool != 0 || p.n_bmax < 2 * p.n_bavg ||
      p.n_bavg < p.n_pool)
    return LSA_ERR_INVALID_ARG;
  if (p.select_mode < LSA_SEM_SELECT_ROW || p.select_mode > LSA_SEM_SELECT_FORCE_OVERFLOW) return LSA_ERR_INVALID_ARG;
  if (d_idx != 64) return LSA_ERR_UNSUPPORTED;
  if (p.n_cluster / p.n_pool > lsa::SEM_MAX_POOL_KEYS || p.n_cluster / p.n_bavg > lsa::SEM_MAX_BUCKETS)
    return LSA_ERR_UNSUPPORTED;
  sp->n_cluster = p.n_cluster;
  sp->n_pool = p.n_pool;
  sp->n_bavg = p.n_bavg;
  sp->n_bmax = p.n_bmax;
  sp->select_mode = p.select_mode;
  return LSA_OK;
}

static lsa_status check_sem_pages(const lsa_semantic_pages* pg, int B, int L_max, int n_blocks, lsa::SemPages* out) {
  *out = lsa::SemPages();
  if (!pg) return LSA_OK;
  if (pg->block_table) {
    if (pg->n_bslots < 1) return LSA_ERR_INVALID_ARG;
    out->block_table = pg->block_table;
    out->n_bslots = pg->n_bslots;
  }
  if (pg->page_table) {
    const int P = pg->page_size;
    if (P < 64 || (P & (P - 1)) != 0 || pg->max_pages < 1 || (long long)pg->max_pages * P != L_max ||
        pg->n_slots < P || pg->n_slots % P != 0 || pg->n_slots > (1LL << 31))
      return LSA_ERR_INVALID_ARG;
    out->page_table = pg->page_table;
    out->page_size = P;
    out->max_pages = pg->max_pages;
    out->n_slots = pg->n_slots;
  }
  (void)B;
  (void)n_blocks;
  return LSA_OK;
}

static lsa_status sem_cluster(const void* k_idx, int32_t B, int32_t L_max, int32_t d_idx,
                              const lsa_semantic_params* prm, const lsa_semantic_pages* pages, int32_t n_blocks,
                              int32_t first_block, int32_t n_update, void* centroids, int32_t* table,
                              int32_t* offsets, void* stream) {
  lsa::SemParams sp;
  if (B < 0 || L_max < 1 || n_blocks < 0 || first_block < 0 || n_update < 0) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_sem_params(prm, d_idx, &sp);
  if (st != LSA_OK) return st;
  if ((long long)first_block + n_update > n_blocks ||
      ((long long)first_block + n_update) * sp.n_cluster > L_max)
    return LSA_ERR_INVALID_ARG;
  lsa::SemPages pg;
  st = check_sem_pages(pages, B, L_max, n_blocks, &pg);
  if (st != LSA_OK) return st;
  if ((long long)B * n_update == 0) return LSA_OK;
  if (!k_idx || !centroids || !table || !offsets) return LSA_ERR_INVALID_ARG;
  return hip_status(lsa::launch_sem_cluster(k_idx, B, L_max, sp, n_blocks, first_block, n_update, centroids, table,
                                            offsets, pg, as_stream(stream)));
}

LSA_API lsa_status lsa_semantic_cluster(const void* k_idx, int32_t B, int32_t L_max, int32_t d_idx,
                                        const lsa_semantic_params* prm, int32_t n_blocks, int32_t first_block,
                                        int32_t n_update, void* centroids, int32_t* table, int32_t* offsets,
                                        void* stream) {
  return sem_cluster(k_idx, B, L_max, d_idx, prm, nullptr, n_blocks, first_block, n_update, centroids, table,
                     offsets, stream);
}

LSA_API lsa_status lsa_semantic_cluster_paged(const void* k_idx, int32_t B, int32_t L_max, int32_t d_idx,
                                              const lsa_semantic_params* prm, const lsa_semantic_pages* pages,
                                              int32_t n_blocks, int32_t first_block, int32_t n_update,
                                              void* centroids, int32_t* table, int32_t* offsets, void* stream) {
  if (!pages) return LSA_ERR_INVALID_ARG;
  return sem_cluster(k_idx, B, L_max, d_idx, prm, pages, n_blocks, first_block, n_update, centroids, table,
                     offsets, stream);
}

LSA_API lsa_status lsa_semantic_select_workspace_size(int32_t B, int32_t n_q, int32_t n_blocks,
                                                      const lsa_semantic_params* prm, size_t* bytes) {
  lsa::SemParams sp;
  if (!bytes || B < 0 || n_q < 0 || n_blocks < 0) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_sem_params(prm, 64, &sp);
  if (st != LSA_OK) return st;
  *bytes = (size_t)B * n_q *
           lsa::sem_select_row_bytes(n_blocks, sp.n_cluster / sp.n_bavg, sp.n_cluster, sp.n_bmax, n_q == 1);
  return LSA_OK;
}

static lsa_status sem_select(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q, int32_t d_idx,
                             const lsa_semantic_params* prm, const lsa_semantic_pages* pages, int32_t L_max,
                             int32_t n_blocks, const void* centroids, const int32_t* table, const int32_t* offsets,
                             int32_t k, int32_t p_top, int32_t n_sink, int32_t n_w, int32_t* idx, int32_t* count,
                             void* ws, size_t ws_bytes, void* stream, void* const* events = nullptr) {
  lsa::SemParams sp;
  if (B < 0 || n_q < 0 || n_blocks < 0 || k < 1 || p_top < 1 || n_sink < 0 || n_w < 0) return LSA_ERR_INVALID_ARG;
  lsa_status st = check_sem_params(prm, d_idx, &sp);
  if (st != LSA_OK) return st;
  if (k > lsa::SEM_MAX_K || p_top > lsa::SEM_MAX_P) return LSA_ERR_UNSUPPORTED;
  lsa::SemPages pg;
  st = check_sem_pages(pages, B, L_max, n_blocks, &pg);
  if (st != LSA_OK) return st;
  if ((long long)n_sink + k + n_w > (1LL << 30)) return LSA_ERR_INVALID_ARG;
  if ((long long)B * n_q == 0) return LSA_OK;
  if (!q_idx || !q_pos || !idx || !count || (n_blocks > 0 && (!centroids || !table || !offsets)))
    return LSA_ERR_INVALID_ARG;
  if (((uintptr_t)ws) % 16 != 0) return LSA_ERR_WORKSPACE;
  const size_t row = lsa::sem_select_row_bytes(n_blocks, sp.n_cluster / sp.n_bavg, sp.n_cluster, sp.n_bmax, n_q == 1);
  if (!ws || ws_bytes < (size_t)B * row) return LSA_ERR_WORKSPACE;
  lsa::SemSelectArgs a;
  a.q_idx = q_idx;
  a.q_pos = q_pos;
  a.B = B;
  a.n_q = n_q;
  a.sp = sp;
  a.NB = n_blocks;
  a.cent = centroids;
  a.table = table;
  a.offs = offsets;
  a.k = k;
  a.p_top = p_top;
  a.n_sink = n_sink;
  a.n_w = n_w;
  a.idx = idx;
  a.count = count;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  a.pages = pg;
  a.events = events;
  return hip_status(lsa::launch_sem_select(a, as_stream(stream)));
}

LSA_API lsa_status lsa_semantic_select(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q, int32_t d_idx,
                                       const lsa_semantic_params* prm, int32_t n_blocks, const void* centroids,
                                       const int32_t* table, const int32_t* offsets, int32_t k, int32_t p_top,
                                       int32_t n_sink, int32_t n_w, int32_t* idx, int32_t* count, void* ws,
                                       size_t ws_bytes, void* stream) {
  return sem_select(q_idx, q_pos, B, n_q, d_idx, prm, nullptr, 0, n_blocks, centroids, table, offsets, k, p_top,
                    n_sink, n_w, idx, count, ws, ws_bytes, stream);
}

LSA_API lsa_status lsa_semantic_select_paged(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q,
                                             int32_t d_idx, const lsa_semantic_params* prm,
                                             const lsa_semantic_pages* pages, int32_t L_max, int32_t n_blocks,
                                             const void* centroids, const int32_t* table, const int32_t* offsets,
                                             int32_t k, int32_t p_top, int32_t n_sink, int32_t n_w, int32_t* idx,
                                             int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  if (!pages) return LSA_ERR_INVALID_ARG;
  return sem_select(q_idx, q_pos, B, n_q, d_idx, prm, pages, L_max, n_blocks, centroids, table, offsets, k, p_top,
                    n_sink, n_w, idx, count, ws, ws_bytes, stream);
}

LSA_API lsa_status lsa_semantic_select_timed(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q,
                                             int32_t d_idx, const lsa_semantic_params* prm, int32_t n_blocks,
                                             const void* centroids, const int32_t* table, const int32_t* offsets,
                                             int32_t k, int32_t p_top, int32_t n_sink, int32_t n_w, int32_t* idx,
                                             int32_t* count, void* ws, size_t ws_bytes, void* stream,
                                             void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2]) return LSA_ERR_INVALID_ARG;
  return sem_select(q_idx, q_pos, B, n_q, d_idx, prm, nullptr, 0, n_blocks, centroids, table, offsets, k, p_top,
                    n_sink, n_w, idx, count, ws, ws_bytes, stream, events);
}
