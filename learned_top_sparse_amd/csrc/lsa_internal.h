// lsa_internal.h -- host-side launcher interface between the C ABI (lsa_api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

// Thresholded selection of flat rows (prefill): each row's threshold and state, and
// its candidate list, in the workspace lsa_forward carves out.
//   rstate: 0 = list row (its entries with score >= theta are appended to its list),
//           1 = table row (short row: its scores go to the score table),
//           2 = list row whose list fell short of k or overflowed cap (the score
//               table path redoes it).
struct ThrArgs {
  const int32_t* theta;
  int32_t* rstate;
  int32_t* cnt;     // entries appended to the row's list (may exceed cap)
  int32_t* lslot;   // [rows][cap]
  int32_t* lscore;  // [rows][cap]
  int cap;
  int row_min;      // rows of at most row_min keys keep the score table
};

// Paged caches: pool row of key j of sequence b (page_table == nullptr: contiguous).
struct Pages {
  const int32_t* page_table;  // [B, max_pages]
  int page_log2, max_pages, n_pages;
};

struct IdxArgs {
  const int8_t* q_idx;
  const int8_t* k_idx;
  const int32_t* w;
  int w_per_query;
  const int32_t* q_pos;
  const int32_t* kept;  // nullptr = flat
  int block_size, n_keep;
  int B, n_q, L_max, H_I, d_I;
  int32_t* scores;
  long long ld;
  int span;        // keys per workgroup span (flat)
  bool use_direct; // flat scores with one query per workgroup (decode-shaped)
  // optional (direct flat only): leave each span's share of the row's selection
  // state -- its coarse score histogram and candidate list -- in the decode
  // selection's workspace (dec_sel_layout) instead of writing the score table
  int* sel_base;
  long long sel_rec_ints;
  int sel_parts, sel_lcap;
  int k_top;
  // flat, many queries (idx_flat_kernel):
  int stride;                  // slot j scores key j * stride (0 or 1: every key)
  ThrArgs thr;                 // thr.theta != nullptr: append candidates instead of writing the table
  const int32_t* tile_filter;  // optional: only query tiles holding a row of state 2
  int row_min;                 // only query tiles holding a row of more than row_min keys (0: all)
  // paged caches (decode selection only): k_idx is a pool of n_pages pages of
  // 2^page_log2 keys; key j of sequence b is in page page_table[b * max_pages + (j >> page_log2)]
  Pages pages;
  // two-stage token stage (block sizes a multiple of 64): the chunk-interleaved copy of
  // k_idx (launch_kidx_interleave), or nullptr to read k_idx itself
  const int8_t* k_il;
};

// Block candidates of decode-shaped rows: the scoring workgroup of span s (span blocks)
// of row r leaves the best min(cap, its blocks) of its span by (score desc, block asc), in
// block order: key[(r * spans + s) * cap + i] (int64 score), blk[...] (block), cnt[r * spans + s].
struct BlkCand {
  long long* key;
  int* blk;
  int* cnt;
  int spans, span, cap;
};

// Thresholded keep of long block rows (block modes, chunks of at least 8 queries per
// sequence), the flat rows' thresholded selection over int64 block scores: a sample of
// every blk_thr_stride(n_keep)-th block gives each row a threshold that about
// 2 (n_keep - 1) of its blocks reach (about BLK_THR_ABOVE samples lie above it); the
// block scan appends those blocks to the row's list (at most blk_thr_cap(n_keep)); the
// exact keep is taken from the list, and rows whose list fell short of n_keep - 1 or
// overflowed are scored again into the score table and kept from there.
struct BlkThr {
  long long* theta;   // [rows]
  int32_t* rstate;    // [rows] 0 list row, 1 table row, 2 list fell short or overflowed
  int32_t* cnt;       // [rows] blocks appended to the list (may exceed cap)
  int32_t* lblk;      // [rows][cap]
  long long* lscore;  // [rows][cap]
  int cap;
  // query tiles (8 queries of one sequence: b * n_qtiles + i / 8) holding a row in
  // state 2, each once: tflag [n_tiles] marks them, tlist [n_tiles] lists them, tcnt [1]
  int32_t* tflag;
  int32_t* tlist;
  int32_t* tcnt;
};
constexpr int BLK_THR_QT = 8;          // queries per tile of the block scoring
constexpr int BLK_THR_FB_SLOTS = 64;   // tiles the fallback scoring takes at once
constexpr int BLK_THR_ABOVE = 32;
constexpr int BLK_THR_MAX_SAMPLES = 8192;  // a row's samples, in registers of one workgroup
constexpr int BLK_THR_MAX_B = 131072;      // the list keep's bitmaps of block positions
constexpr int BLK_THR_MIN_STRIDE = 16;     // sampling costs at most 1/16 of the scan
inline int blk_thr_cap(int n_keep) { return 4 * n_keep; }
inline int blk_thr_stride(int n_keep) {
  const int st = 2 * (n_keep - 1) / BLK_THR_ABOVE;
  return st > 1 ? st : 1;
}
// Rows of at most this many scored blocks keep the score table: below it the table's
// round trip (8 bytes written and 16 read per block) costs less than the list path's
// fixed share per row (measured on MI355X at n_keep = 512: rows of 4K-8K blocks ran
// slower through lists, rows of 62K blocks 7 % faster per step).
inline int blk_thr_row_min(int n_keep) { return 8 * n_keep > 16384 ? 8 * n_keep : 16384; }

struct BlkArgs {
  const int8_t* q_idx;
  const int8_t* limbs;
  const int32_t* w;
  int w_per_query;
  const int32_t* q_pos;
  int B, n_q, n_blocks, L_max, H_I, d_I, block_size;
  long long* bscores;
  long long ld;
  int span;
  BlkCand cand;  // decode-shaped rows: candidates instead of the score table (key == nullptr: table)
  // prefill-shaped rows only:
  int stride;    // > 1: score blocks 0, stride, 2 stride, ... into column m / stride (the sample)
  int mode;      // 0 every row into the table; 1 thresholded scan (thr); 2 rows in state 2 only
  BlkThr thr;
};

struct TopkArgs {
  const int32_t* scores;
  long long ld;
  const int32_t* q_pos;
  const int32_t* kept;
  int block_size, n_keep;
  int B, n_q, L_max, k;
  int32_t* idx;
  int32_t* count;
  void* ws;          // optional: enables the several-workgroups-per-row path
  size_t ws_bytes;
  bool hist_ready;   // the indexer built the rows' selection state in ws (dec_sel_layout)
  const int32_t* row_state;  // optional (flat): only rows whose state (ThrArgs) is not 0
  Pages pages;               // hist_ready with paged caches: the lists receive pool rows
};

struct BlkSelArgs {
  const long long* bscores;
  long long ld;
  const int32_t* q_pos;
  int B, n_q, n_blocks, block_size, n_keep;
  int32_t* kept;
  BlkCand cand;  // key != nullptr: merge the scoring workgroups' candidates instead
  const int32_t* rstate;  // non-null: rows in state 0 (kept from their lists) are skipped
};

// waves per sparse-attention workgroup (each with its own 32-key tile state)
constexpr int ATTN_WAVES = 4;
// keys per workgroup of the direct (decode-shaped) flat indexer that writes a score table
constexpr int DIRECT_SPAN = 4096;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  int B, n_q, L_max, H_q, d, k_top;
  long long kv_pool;  // > 0: k, v are pools of kv_pool rows and idx holds pool rows
  float scale;
  int n_split;
  void* out;
  float* lse;
  float* ws;  // n_split > 1: partial outputs [rows, n_split, H_q, d] then lse [rows, n_split, H_q]
};

hipError_t launch_index_scores(const IdxArgs& a, hipStream_t st);
hipError_t launch_block_reps(const int8_t* k_idx, int B, int L_max, int d_I, int bs, int n_blocks,
                             int32_t* reps, hipStream_t st);
hipError_t launch_block_limbs(const int32_t* reps, int B, int n_blocks, int d_I, int8_t* limbs,
                              hipStream_t st);
hipError_t launch_block_scores(const BlkArgs& a, hipStream_t st);
// Candidate layout of decode-shaped block rows (rows of fewer than 8 queries per sequence)
// carved from `region` (region_bytes); false if it does not fit or the rows are not
// decode-shaped (then the score table is used).
bool blk_cand_layout(long long rows, int n_q, int n_blocks, int n_keep, void* region, size_t region_bytes,
                     BlkCand* c);
// block-key cache (the limbs of the representatives) of blocks [m0, m0 + n_upd)
hipError_t launch_block_cache(const int8_t* k_idx, int B, int L_max, int d_I, int bs, int n_blocks, int m0,
                              int n_upd, int8_t* limbs, hipStream_t st, const Pages& pg = Pages{});
// pooled blocks: index lists = the keys of the kept blocks a query may see
hipError_t launch_expand(const int32_t* kept, const int32_t* q_pos, long long rows, int bs, int n_keep, int k,
                         int32_t* idx, int32_t* count, hipStream_t st, const Pages& pg = Pages{}, int n_q = 1);
hipError_t launch_block_select(const BlkSelArgs& a, hipStream_t st);
// thresholded block keep: each row's threshold from its sampled scores (samp: ld_s per
// row; mode 0 sampled quantile, 1 above every score, 2 below every score) ...
hipError_t launch_blk_thresholds(const long long* samp, long long ld_s, const int32_t* q_pos, int B, int n_q,
                                 int n_blocks, int bs, int n_keep, int stride, int row_min, int mode,
                                 const BlkThr& t, hipStream_t st);
// ... and the exact keep of the list rows (rows whose list fell short or overflowed: state 2,
// their tiles listed for the fallback scoring)
hipError_t launch_blk_list_keep(const int32_t* q_pos, int B, int n_q, int n_blocks, int bs, int n_keep,
                                const BlkThr& t, int32_t* kept, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// chunk-interleaved copy of the index keys of B sequences for the token stage: bytes, and
// the kernel that writes it (paged caches through pg)
size_t kidx_interleave_bytes(int B, int L_max, int d_I);
hipError_t launch_kidx_interleave(const int8_t* k_idx, int B, int L_max, int d_I, const Pages& pg, int8_t* out,
                                  hipStream_t st);
// two-stage token stage and its top-k in one kernel (rows of at most KSEL_SLOTS kept slots)
constexpr int KSEL_SLOTS = 8192;
hipError_t launch_kept_select(const IdxArgs& a, int k, int32_t* idx, int32_t* count, hipStream_t st);
// workspace that lets lsa_topk split each row over several workgroups (0 = not used)
size_t topk_ws_bytes(long long rows, int L_max);
// Decode selection: the indexer builds each row's selection state (histogram, one
// candidate list per span) and one workgroup per row finishes the top-k from it.
// Layout of `rows` rows of L_max keys and top-k size k: spans per row, list
// capacity, ints per record.  Returns false where the path does not apply.
struct DecLayout {
  int parts, lcap;
  long long rec_ints;  // ints per (row, span) record
};
bool dec_sel_layout(long long rows, int L_max, int k, DecLayout* out);
// workspace of the decode selection (0 where it does not apply); a chunk of fewer
// rows of the same L_max and k never needs more per row
size_t dec_sel_ws_bytes(long long rows, int L_max, int k);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t st);

// Thresholded selection of flat rows (prefill rows longer than thr_cap(k) keys): a
// sample of every thr_stride(k)-th key gives each row a threshold that about 2k of
// its entries reach -- about THR_ABOVE samples lie above it, so the count is known to
// +-1/sqrt(THR_ABOVE) -- the scan appends those entries to the row's list (at most
// thr_cap(k)); the exact top-k is taken from the list, and rows whose list fell short
// of k or overflowed go through the score table.
constexpr int THR_ABOVE = 64;       // sampled entries expected above a row's threshold
constexpr int THR_MAX_K = 2048;     // list rows hold at most 4 * 2048 entries (LDS of the list top-k)
constexpr int THR_MAX_L = 524288;   // the list top-k's slot bitmap (64 KB)
inline int thr_cap(int k) { return 4 * k; }
// Rows of at most 8k keys keep the score table: below that the table's round trip
// costs less than the sample, the list and its selection (measured on MI355X: rows of
// 8K..16K keys at k = 2048 ran 7 % slower through lists, rows past 24K keys faster).
inline int thr_row_min(int k) { return 8 * k; }
// 2k entries above the threshold for THR_ABOVE samples: one sample per 2k / THR_ABOVE keys
inline int thr_stride(int k) { return k * 2 / THR_ABOVE > 1 ? k * 2 / THR_ABOVE : 1; }
// modes of launch_thresholds: 0 sampled quantile; 1 threshold above every score (all
// list rows fall short); 2 threshold below every score (list rows overflow)
hipError_t launch_thresholds(const int32_t* samp, long long ld_s, const int32_t* q_pos, long long rows, int L_max,
                             int k, int stride, int mode, const ThrArgs& t, hipStream_t st);
// exact top-k of the list rows; marks rows whose list fell short or overflowed (state 2)
hipError_t launch_list_topk(const int32_t* q_pos, long long rows, int L_max, int k, const ThrArgs& t,
                            int32_t* idx, int32_t* count, int n_q, const Pages& pg, hipStream_t st);

// ---- flat semantic search (Ward bucket cache, centroid scoring, top-p, expansion)
struct SemParams {
  int n_cluster, n_pool, n_bavg, n_bmax;
  int select_mode;  // lsa_semantic_params.select_mode
};
struct SemPages {
  const int32_t* block_table = nullptr;  // [B, NB] cache slot of each cluster block (null: b * NB + t)
  int n_bslots = 0;
  const int32_t* page_table = nullptr;   // [B, max_pages] pool page of each page of keys (null: contiguous)
  int page_size = 0, max_pages = 0;
  long long n_slots = 0;                 // rows of the key pools
};
struct SemSelectArgs {
  const void* q_idx;       // bf16 [B, n_q, 64]
  const int32_t* q_pos;    // [B, n_q]
  int B, n_q;
  SemParams sp;
  int NB;                  // cluster blocks the cache holds per sequence
  const void* cent;
  const int32_t* table;
  const int32_t* offs;
  int k, p_top, n_sink, n_w;
  int32_t* idx;            // [B, n_q, n_sink + k + n_w]
  int32_t* count;          // [B, n_q]
  void* ws;
  size_t ws_bytes;
  SemPages pages;
  void* const* events = nullptr;  // optional: 3 caller-made HIP events (scan start, scan end, end)
};
constexpr int SEM_MAX_POOL_KEYS = 128;  // pool keys of a cluster block
constexpr int SEM_MAX_BUCKETS = 64;     // buckets of a cluster block
constexpr int SEM_MAX_P = 2048;
constexpr int SEM_MAX_K = 4096;
hipError_t launch_sem_cluster(const void* k_idx, int B, int L_max, const SemParams& sp, int NB, int first_block,
                              int n_update, void* cent, int32_t* table, int32_t* offs, const SemPages& pages,
                              hipStream_t st);
size_t sem_select_row_bytes(int NB, int m, int n_cluster, int n_bmax, bool decode);
hipError_t launch_sem_select(const SemSelectArgs& a, hipStream_t st);

}  // namespace lsa
