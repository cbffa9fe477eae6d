/*
 * lsa.h -- C ABI of the learned top-k sparse attention hot path on MI355X (gfx950).
 *
 * The path (indexer -> exact top-k -> sparse attention):
 *   1. a lightweight int8 indexer scores every causally preceding key of each query;
 *   2. an exact per-query top-k keeps k keys (ties: lowest key index);
 *   3. bf16 attention with an fp32 online softmax runs over only those keys;
 *   optionally a two-stage indexer first keeps the best key blocks and scores
 *   tokens only inside them.
 *
 * Sources (pages on learned sparse attention):
 *   [LSA]  "Latent Sparse Attention (LSA)" (paperpeel.com/paper/2610.42147):
 *          §2 "Sparse Attention" -- cost O(Tk) to prefill, O(k) per decoded token;
 *          §2.1 "Design Choices", "Token Sparse Attention" -- a cheap, narrow,
 *          low-precision scorer rates every earlier key;
 *          §3.1 "Pooling" -- a pooled key is the sum of consecutive index keys;
 *          §3.2 "Attention" -- one index list J_i serves every query head;
 *          App. F.1 "Selection by threshold" -- packed (score, inverted id) keys:
 *          better score first, lower id first at equal score; order of J_i is free;
 *          App. F.1 "Attention kernels" -- J_i is a row of int32 cache slots padded
 *          with -1, read by attention like a page table;
 *          App. F.1 "CUDA graphs" -- decode steps are replayed from graphs, so a
 *          step must not read anything back on the host.
 *   [HISA] summary "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 *          Attention" (theflow.svmpsp.dev related-papers page): block-level coarse
 *          filter, then the token indexer only inside the kept blocks.
 *   [HyTopK] HyScale summary on the same page: exact per-query top-k.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE memory owned by the caller (e.g. torch tensors' data_ptr),
 *     contiguous row-major, at least 16-byte aligned.  The library never allocates,
 *     frees or synchronises; scratch memory is the caller's workspace `ws` of
 *     `ws_bytes`, sized by the matching *_workspace_size call.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream).  Outputs are valid once the caller synchronises;
 *     inputs must not change before then.  No call reads anything back to the
 *     host, so every call can be captured in a HIP graph.
 *   - Errors: arguments are validated on the host first; on error the call returns
 *     a negative status, launches nothing and leaves outputs untouched.  A failed
 *     launch returns LSA_ERR_HIP.  Device-side faults surface at the caller's sync.
 *   - q_pos[b*n_q + i] is the absolute position p of query i of sequence b; it
 *     sees keys 0..p (its own key included).  Keys j >= L_max are never read:
 *     p is clipped to L_max-1, and p < 0 gives a query with no candidates.
 *   - Thread safety: reentrant, no global state.  Concurrent calls need distinct
 *     workspaces.
 *   - Exactness preconditions (device data cannot be checked on the host):
 *     |w_h| < 2^23, and |sum_h w_h * max(0, q_h.k_j)| < 2^31 for token scores
 *     (true for int8 in [-64, 64], 1 <= w <= 16, H_I <= 64, d_I <= 128); block
 *     scores are int64 and need |sum| < 2^63.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int lsa_status;
enum {
  LSA_OK = 0,
  LSA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes */
  LSA_ERR_UNSUPPORTED = -2, /* shape outside the compiled variants (see each call) */
  LSA_ERR_WORKSPACE = -3,   /* ws too small (query *_workspace_size) or misaligned */
  LSA_ERR_HIP = -4,         /* a kernel launch failed */
  LSA_ERR_INTERNAL = -5
};

enum { LSA_MODE_PREFILL = 0, LSA_MODE_DECODE = 1 };

/* Human-readable name of a status code (static storage). */
const char* lsa_status_string(lsa_status s);
/* Library version: major*10000 + minor*100 + patch. */
int lsa_version(void);

/*
 * Token-indexer scores ([LSA] §2.1 "Token Sparse Attention"; the weighted-ReLU
 * form used here is this library's reading of the indexer the pages leave open):
 *     S[b,i,j] = sum_h w_h * max(0, sum_d q_idx[b,i,h,d] * k_idx[b,j,d])
 * exact in int32, for every key j <= q_pos[b,i] (entries for later keys are
 * left unspecified; they may or may not be written).
 *   q_idx  int8  [B, n_q, H_I, d_I]     index queries (H_I heads each)
 *   k_idx  int8  [B, L_max, d_I]        one index key per token, shared by heads
 *   w      int32 [H_I] (w_per_query=0) or [B, n_q, H_I] (w_per_query=1)
 *   q_pos  int32 [B, n_q]
 *   kept_blocks int32 [B, n_q, n_keep] or NULL.
 *     NULL: flat mode, scores[(b*n_q+i)*ld_scores + j] for keys j.
 *     non-NULL: two-stage token stage ([HISA]); only keys of the listed blocks
 *     (block m = keys m*block_size .. m*block_size+block_size-1; -1 = unused
 *     entry) are scored, into compact slots:
 *       scores[(b*n_q+i)*ld_scores + s], key(s) = kept[s / block_size]*block_size
 *                                                + s % block_size,
 *     for s < n_keep*block_size (ld_scores >= n_keep*block_size).  Slots whose
 *     block is -1 or whose key is past q_pos are left unspecified.
 * Supported: d_I in {64, 128}; 1 <= H_I <= 64; ld_scores >= L_max (flat).
 * Exactness: each w_h must lie in [-2^23, 2^23) (the weight product uses 24-bit
 * signed multiplies; a ReLU'd dot is at most 2^21) and every score must fit in
 * int32; weights are device data and are not checked.
 * No workspace.
 */
lsa_status lsa_index_scores(const int8_t* q_idx, const int8_t* k_idx, const int32_t* w,
                            int32_t w_per_query, const int32_t* q_pos,
                            const int32_t* kept_blocks, int32_t block_size, int32_t n_keep,
                            int32_t B, int32_t n_q, int32_t L_max, int32_t H_I, int32_t d_I,
                            int32_t* scores, int64_t ld_scores, void* stream);

/*
 * Block representatives ([LSA] §3.1 "Pooling": a pooled key is the sum of its
 * consecutive index keys; [HISA] scores such block summaries):
 *     reps[b,m,:] = sum_{t < block_size} k_idx[b, m*block_size + t, :]   (int32)
 * for m < n_blocks; requires n_blocks*block_size <= L_max (complete blocks only).
 * Supported: d_I in {64, 128}; 1 <= block_size <= 128.  No workspace.
 */
lsa_status lsa_block_reps(const int8_t* k_idx, int32_t B, int32_t L_max, int32_t d_I,
                          int32_t block_size, int32_t n_blocks, int32_t* reps, void* stream);

/*
 * Block-key cache of the block modes of lsa_forward (two_stage = 1 or 2): for blocks
 * m in [first_block, first_block + n_update) of every sequence, the representative
 * r = sum of the block's block_size index keys ([LSA] §3.1 "Pooling"), stored as two
 * int8 parts r = 128 * hi + lo, lo in [-64, 63]:
 *     block_keys[b, m, 0, :] = hi,  block_keys[b, m, 1, :] = lo   (int8 [B, n_blocks, 2, d_I])
 * A serving loop builds it once and then updates only the block a new token
 * completes (n_update = 1).  Requires (first_block + n_update) * block_size <= L_max.
 * Supported: d_I in {64, 128}; 1 <= block_size <= 128.  No workspace.
 */
lsa_status lsa_block_cache(const int8_t* k_idx, int32_t B, int32_t L_max, int32_t d_I, int32_t block_size,
                           int32_t n_blocks, int32_t first_block, int32_t n_update, int8_t* block_keys,
                           void* stream);
/* The same cache for index keys in a paged pool ([LSA] App. F.1 "Attention kernels":
 * caches are read through page tables; reading as lsa_forward_args.page_table below):
 * k_idx_pool int8 [n_slots, d_I], page_table int32 [B, max_pages], pages of page_size
 * keys (a power of two >= 64; n_slots a multiple of it, at most 2^31).  Logical key j
 * of sequence b is pool row page_table[b][j / page_size] * page_size + j % page_size;
 * page ids outside [0, n_slots / page_size) are clamped into it.  The cache itself is
 * per sequence, [B, n_blocks, 2, d_I] as above; the blocks cover logical keys, so
 * (first_block + n_update) * block_size <= max_pages * page_size. */
lsa_status lsa_block_cache_paged(const int8_t* k_idx_pool, int64_t n_slots, const int32_t* page_table,
                                 int32_t page_size, int32_t max_pages, int32_t B, int32_t d_I, int32_t block_size,
                                 int32_t n_blocks, int32_t first_block, int32_t n_update, int8_t* block_keys,
                                 void* stream);

/*
 * Two-stage block prefilter ([HISA]; [LSA] §2.2 "Related Work": score blocks
 * first, then only the keys inside the selected blocks).  For each query with
 * own block o = floor(q_pos/block_size):
 *     BS[m] = sum_h w_h * max(0, q_h . reps[m])   (int64), for blocks m < o,
 *     kept  = {o} U the best min(n_keep-1, o) blocks by (BS desc, m asc),
 * written ascending into kept_blocks[b,i,0..] and padded with -1 to n_keep.
 *   reps          int32 [B, n_blocks, d_I] from lsa_block_reps (n_blocks must
 *                 cover every own block: floor(max q_pos / block_size) <= n_blocks)
 *   block_scores  optional int64 [B, n_q, n_blocks] output (entries m < o valid) or NULL
 * Supported: d_I in {64,128}; 1 <= H_I <= 64; 1 <= block_size <= 128;
 * 1 <= n_keep <= 256; n_blocks <= 65536.  Workspace: lsa_block_prefilter_workspace_size.
 */
lsa_status lsa_block_prefilter_workspace_size(int32_t B, int32_t n_q, int32_t n_blocks,
                                              int32_t d_I, size_t* bytes);
lsa_status lsa_block_prefilter(const int8_t* q_idx, const int32_t* reps, const int32_t* w,
                               int32_t w_per_query, const int32_t* q_pos, int32_t B, int32_t n_q,
                               int32_t n_blocks, int32_t H_I, int32_t d_I, int32_t block_size,
                               int32_t n_keep, int32_t* kept_blocks, int64_t* block_scores,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * Exact per-query top-k ([HyTopK]; tie rule of [LSA] App. F.1 "Selection by
 * threshold"): idx[b,i,:] = the min(k, n_cand) candidates with the largest
 * scores, equal scores ranked by lower key index first, written in ASCENDING
 * key order and padded with -1 ([LSA] App. F.1 "Attention kernels").
 * Candidates: flat mode (kept_blocks == NULL) keys 0..min(q_pos, L_max-1) with
 * scores[(b*n_q+i)*ld_scores + j]; two-stage mode the compact slots written by
 * lsa_index_scores with kept_blocks (keys <= q_pos and < L_max of listed blocks).
 *   count  optional int32 [B, n_q] = number of indices written (or NULL).
 * Supported: 1 <= k <= 4096.  Workspace: lsa_topk_workspace_size returns a
 * nonzero size when few long flat rows are better split over several
 * workgroups each (decode-shaped calls); with a smaller or NULL workspace the
 * one-workgroup-per-row algorithm runs instead.  Results are identical.
 */
lsa_status lsa_topk_workspace_size(int32_t B, int32_t n_q, int32_t L_max, int32_t k, size_t* bytes);
lsa_status lsa_topk(const int32_t* scores, int64_t ld_scores, const int32_t* q_pos,
                    const int32_t* kept_blocks, int32_t block_size, int32_t n_keep,
                    int32_t B, int32_t n_q, int32_t L_max, int32_t k,
                    int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse attention over the index lists ([LSA] §3.2 "Attention": one list per
 * query shared by all heads; §2: O(k) per query):
 *     out[b,i,h,:] = sum_{j in J} softmax_j(scale * q[b,i,h,:].k[b,j,:]) v[b,j,:]
 * with J = the entries of idx[b,i,:] in [0, L_max) (-1 and out-of-range entries
 * are skipped; order does not matter).  bf16 MFMA products, fp32 online softmax,
 * bf16 output (round to nearest even).  An empty list gives out = 0, lse = -inf.
 *   q   bf16 [B, n_q, H_q, d];  k, v  bf16 [B, L_max, d] (one KV head)
 *   idx int32 [B, n_q, k]
 *   out bf16 [B, n_q, H_q, d];  lse optional fp32 [B, n_q, H_q] (natural log) or NULL
 * n_split > 1 splits each list into n_split parts merged by log-sum-exp (the
 * split-KV form used for decode); n_split = 0 picks automatically.
 * Supported: d = 128; 1 <= H_q <= 16; 1 <= k <= 65536.
 * Workspace: lsa_sparse_attn_workspace_size (0 when n_split resolves to 1).
 */
lsa_status lsa_sparse_attn_workspace_size(int32_t B, int32_t n_q, int32_t H_q, int32_t d, int32_t k,
                                          int32_t n_split, size_t* bytes);
lsa_status lsa_sparse_attn(const void* q, const void* k, const void* v, const int32_t* idx,
                           int32_t B, int32_t n_q, int32_t L_max, int32_t H_q, int32_t d, int32_t k_top,
                           float scale, int32_t n_split, void* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* The same attention over shared K/V pools (paged caches): k_pool, v_pool bf16
   [n_slots, d] hold every sequence's keys and idx entries are pool rows (entries outside
   [0, n_slots) and -1 are skipped) -- the lists of lsa_forward or lsa_semantic_select_paged
   with a page table.  Same support and workspace as lsa_sparse_attn. */
lsa_status lsa_sparse_attn_pool(const void* q, const void* k_pool, const void* v_pool, const int32_t* idx,
                                int32_t B, int32_t n_q, int64_t n_slots, int32_t H_q, int32_t d, int32_t k,
                                float scale, int32_t n_split, void* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * The whole path in one call ([LSA] §2; [HISA] for two_stage):
 *   PREFILL flat:      per chunk of query rows: index_scores -> topk -> sparse_attn
 *   PREFILL two_stage: block_reps (once) -> block_prefilter -> index_scores (kept)
 *                      -> topk (kept) -> sparse_attn
 *   DECODE:            as PREFILL with one query per sequence (n_q = 1); the
 *                      caller appends the new token's k/v/k_idx first and passes
 *                      q_pos = its position.  Attention is split over keys.
 * Score rows are materialised chunk by chunk in the workspace; chunk_rows = 0
 * picks the largest chunk that fits ws_bytes.
 */
typedef struct lsa_forward_args {
  int32_t mode;          /* LSA_MODE_PREFILL or LSA_MODE_DECODE */
  int32_t two_stage;     /* 0 flat; 1 block prefilter then tokens; 2 pooled blocks (below) */
  const int8_t* q_idx;   /* int8 [B, n_q, H_I, d_I] */
  const int8_t* k_idx;   /* int8 [B, L_max, d_I] */
  const int32_t* w;      /* int32 [H_I] or [B, n_q, H_I] */
  int32_t w_per_query;
  const int32_t* q_pos;  /* int32 [B, n_q] */
  const void* q;         /* bf16 [B, n_q, H_q, d] */
  const void* k;         /* bf16 [B, L_max, d] */
  const void* v;         /* bf16 [B, L_max, d] */
  int32_t B, n_q, L_max, H_I, d_I, H_q, d, k_top;
  int32_t block_size, n_keep; /* two-stage only */
  float scale;           /* softmax scale, e.g. 1/sqrt(d) */
  int32_t attn_split;    /* 0 = automatic */
  int64_t chunk_rows;    /* query rows per score chunk; 0 = automatic */
  int32_t* idx;          /* out int32 [B, n_q, k_top] */
  int32_t* count;        /* out int32 [B, n_q] or NULL */
  void* out;             /* out bf16 [B, n_q, H_q, d] */
  float* lse;            /* out fp32 [B, n_q, H_q] or NULL */
  int32_t* kept_blocks;  /* out int32 [B, n_q, n_keep] (two-stage) or NULL */
  /* Optional stage timing: hipEvent_t handles created by the caller.  lsa_forward
     records stage_events[0] on `stream` before its first launch and
     stage_events[e] after its e-th stage, in launch order (lsa_forward_stages
     lists the stages).  n_stage_events must be at least 1 + that count, else
     LSA_ERR_INVALID_ARG and nothing is launched.  NULL: no events. */
  void* const* stage_events;
  int32_t n_stage_events;
  /* Selection of flat rows of at least 8 queries per sequence (prefill):
     LSA_SELECT_AUTO (0): rows longer than 8*k_top keys (k_top <= 2048, L_max <= 524288)
       take the thresholded selection -- a sample of every row's keys gives it a
       threshold, the indexer keeps only the entries that reach it, and the exact
       top-k is taken from those; a row whose kept entries fall short of k_top or
       overflow 4*k_top goes through the score table instead.  Other rows use the
       score table.  The results are the same either way.
     Block modes (two_stage > 0, chunks of at least 8 queries per sequence) choose the
     block keep the same way: with AUTO, rows over max(8*n_keep, 16384) blocks (n_keep
     from 257 to 2048, at most 131072 blocks) take the thresholded keep -- every
     (2*(n_keep-1)/32)-th block scored as a sample gives each row a threshold, the
     block scan lists the blocks that reach it, and the kept blocks are taken from the
     list; a row whose list falls short of n_keep-1 or overflows 4*n_keep is scored
     again into the block score table.  Other rows use the table.  The results are the
     same either way.
     LSA_SELECT_TABLE (1): every row through the score table.
     LSA_SELECT_FORCE_SHORT (2), LSA_SELECT_FORCE_OVERFLOW (3): as AUTO, but every
       thresholded row's threshold is set above (below) all of its scores, so every
       such row takes the fallback -- for testing that path. */
  int32_t select_mode;
  /* Paged caches (serving-style decode; [LSA] App. F.1 "Attention kernels": the index
     list is read like a page table).  page_table != NULL: k_idx, k and v are pools of
     n_slots rows shared by all sequences (int8 [n_slots, d_I], bf16 [n_slots, d]),
     and logical key j of sequence b is pool row
         page_table[b * max_pages + j / page_size] * page_size + j % page_size.
     L_max must equal max_pages * page_size; page_size is a power of two >= 64 and
     n_slots a multiple of it (at most 2^31).  Page ids outside [0, n_slots / page_size)
     are clamped into that range (no fault; the result is then unspecified).  Selection
     runs on logical keys (ties: lower logical index) and idx receives the pool rows of
     the kept keys, in ascending logical order, -1 padded.  Flat calls: decode and
     prefill chunks alike; a chunk of fewer than 8 queries per sequence must fit its
     decode selection state in the workspace (else LSA_ERR_WORKSPACE).  Block modes:
     the block-key cache covers logical blocks (block_keys from lsa_block_cache_paged,
     or built here through the page table) and kept_blocks holds logical block ids;
     the two-stage token stage must take its one-kernel form (n_keep <= 256 and
     n_keep * block_size <= 8192, else LSA_ERR_UNSUPPORTED).  Sequences of different lengths share a call through q_pos;
     with L_max fixed (one per range of context lengths) the launches keep one shape,
     so a captured HIP graph replays for any positions and page tables.
     page_table == NULL: contiguous caches [B, L_max, ...]. */
  const int32_t* page_table;  /* int32 [B, max_pages] */
  int32_t page_size, max_pages;
  int64_t n_slots;
  /* Block modes: the block-key cache of lsa_block_cache for all L_max / block_size
     blocks, or NULL (then lsa_forward builds it in its workspace, stage block_reps).
     Pooled blocks (two_stage = 2; the "score every block of four keys" indexers of
     [LSA] §2.2 "Related Work" and the LSA page's flat baseline): each query keeps its
     own block and the best n_keep - 1 earlier complete blocks by their block score (as
     two_stage = 1), and its list is every key of those blocks it may see, ascending,
     -1 padded: k_top must equal n_keep * block_size.  Stages block_prefilter ->
     expand -> sparse_attn per chunk. */
  const int8_t* block_keys;
} lsa_forward_args;
enum { LSA_SELECT_AUTO = 0, LSA_SELECT_TABLE = 1, LSA_SELECT_FORCE_SHORT = 2, LSA_SELECT_FORCE_OVERFLOW = 3 };

/* Workspace for lsa_forward.  With a->chunk_rows = 0 it sizes chunks whose per-row
   buffers (score table, sampled scores, candidate lists) come to at most ~8 GiB;
   lsa_forward then uses whatever chunk fits the ws it gets. */
lsa_status lsa_forward_workspace_size(const lsa_forward_args* a, size_t* bytes);
lsa_status lsa_forward(const lsa_forward_args* a, void* ws, size_t ws_bytes, void* stream);
/* Allocation-free lsa_forward, for callers that cannot allocate device memory: code
   under HIP graph capture, serving loops and harnesses that forbid hipMalloc.  Same
   arguments, results and stages as lsa_forward with ws_bytes = LSA_NOALLOC_SCRATCH_BYTES;
   the workspace is a device array of that size inside the library, one per GPU, held
   until the process ends.  The call allocates and frees nothing (device or host-pinned)
   and calls no allocating routine.
     Sizes: chunks are planned to fit the array (as lsa_forward_plan with that ws_bytes);
       a call whose requested chunk_rows, or whose single row, needs more returns
       LSA_ERR_WORKSPACE and launches nothing.  decode_128k (64 sequences of 131073 keys,
       k_top 2048) needs 70.1 MiB and runs as one chunk.
     Device: the current device; `stream` must belong to it.  The array's device address
       is looked up on the first call on each device (one hipGetSymbolAddress), so make
       that first call outside graph capture; later calls only launch kernels.
     Sharing: every call on one GPU uses the same array, so calls that overlap on one GPU
       (other streams, other host threads) race; order them on one stream.  The array
       keeps the last call's contents; no kernel needs it cleared beforehand (each call
       clears what it counts in).
   Errors as lsa_forward; LSA_ERR_HIP also if the array's address cannot be found. */
#define LSA_NOALLOC_SCRATCH_BYTES (128ull << 20)
lsa_status lsa_forward_noalloc(const lsa_forward_args* a, void* stream);
/* The launch plan lsa_forward uses with a workspace of ws_bytes: query rows per
   score chunk (sequences per chunk when n_q == 1) and the attention split count.
   Calling lsa_index_scores / lsa_topk / lsa_sparse_attn chunk by chunk with
   these values (ld_scores = L_max rounded up to 64, or n_keep*block_size for
   two_stage) reproduces lsa_forward's results bit for bit. */
lsa_status lsa_forward_plan(const lsa_forward_args* a, size_t ws_bytes, int64_t* chunk_rows, int32_t* attn_split);

/* Stages of lsa_forward, in launch order, for a workspace of ws_bytes.  A stage is
   one kernel or a short fixed sequence of them:
     BLOCK_REPS       the block-key cache (block modes without block_keys, once per call)
     BLOCK_PREFILTER  block scores and kept blocks of a chunk (block modes)
     EXPAND           pooled blocks: the keys of the kept blocks as the index lists
     INDEX_SELECT     the indexer over a chunk of flat rows of few queries per
                      sequence (fewer than 8) that leaves, instead of the score
                      table, each key span's share of the selection state (coarse
                      score histogram and candidate list); TOPK then finishes each
                      row from it (the decode selection)
     SAMPLE           thresholded selection of flat prefill rows: the indexer over a
                      sample of every row's keys and each row's threshold; then
                      INDEX_SELECT keeps each row's entries that reach it (short
                      rows write the score table) and TOPK takes the exact top-k
                      from them (with the score-table fallback)
     INDEX_SCORES     the indexer over a chunk, writing the score table
     TOPK             the exact top-k of a chunk
     SPARSE_ATTN      sparse attention of a chunk (split-KV combine included)
   Writes min(n, max_codes) codes to `codes` (may be NULL) and n to *n_stages. */
enum {
  LSA_STAGE_BLOCK_REPS = 1,
  LSA_STAGE_BLOCK_PREFILTER = 2,
  LSA_STAGE_INDEX_SELECT = 3,
  LSA_STAGE_INDEX_SCORES = 4,
  LSA_STAGE_TOPK = 5,
  LSA_STAGE_SPARSE_ATTN = 6,
  LSA_STAGE_SAMPLE = 7,
  LSA_STAGE_EXPAND = 8
};
lsa_status lsa_forward_stages(const lsa_forward_args* a, size_t ws_bytes, int32_t* codes, int32_t max_codes,
                              int32_t* n_stages);

/* ---------------------------------------------------------------------------------
 * Flat semantic search ([LSA] §3.1 "Semantic Clustering", §3.2 "Semantic Search",
 * App. F.1 "Kernels").  Index keys and queries are bf16 vectors of d_idx = 64.
 *
 * Cluster blocks are runs of n_cluster consecutive keys.  A complete block's keys are
 * L2 normalised and summed n_pool at a time into pool keys; the pool keys are merged
 * bottom up by Ward's criterion (every round, all pairs of buckets that are each
 * other's cheapest allowed merge merge at once; a merge is allowed while the bucket
 * holds at most n_bmax keys) until m = n_cluster / n_bavg buckets remain.  A bucket's
 * centroid is its normalised key sum, in bf16.  A query (normalised, bf16) scores the
 * centroids of every block before its own, keeps the top p_top buckets (higher score
 * first, then lower bucket id) and expands them, best first, into k long-range keys,
 * skipping keys of the sink (j < n_sink) and of the window (j > p - n_w); its list is
 * the sink, those keys and the window.
 *
 * Every floating-point step that decides which buckets merge or are kept runs in fp32
 * with each operation rounded on its own and sums over the dimensions taken in order,
 * so results are deterministic and reproducible on any machine that rounds the same
 * way (the CPU oracle does).
 */
typedef struct lsa_semantic_params {
  int32_t n_cluster; /* keys per cluster block */
  int32_t n_pool;    /* keys summed into one pool key; divides n_cluster and n_bmax */
  int32_t n_bavg;    /* average keys per bucket; divides n_cluster (m = n_cluster / n_bavg) */
  int32_t n_bmax;    /* largest bucket, in keys; at least 2 * n_bavg (so exactly m buckets form) */
  /* How lsa_semantic_select finds the top-p buckets of decode rows (one query per
   * sequence); the result is the exact top-p in every mode, and prefill rows always rank
   * their whole score row.
   *   LSA_SEM_SELECT_ROW (0): every row ranks its whole score row (one workgroup holds
   *     rows of up to 32768 buckets in registers; longer rows merge spans' top-p).
   *   LSA_SEM_SELECT_THRESHOLD (1): the threshold list of [LSA] App. F.1 "Selection by
   *     threshold", "Flat decode", for rows of more than LSA_SEM_LIST_CAP buckets with
   *     p_top <= LSA_SEM_LIST_CAP / 4: a threshold is set from a sample of the row
   *     (about 2 p_top buckets reach it), the scan lists every bucket at or above it, and
   *     only the list is ranked; a row whose list falls short of p_top or overflows its
   *     LSA_SEM_LIST_CAP entries ranks its whole score row instead.
   *   LSA_SEM_SELECT_FORCE_SHORT (2), LSA_SEM_SELECT_FORCE_OVERFLOW (3): as THRESHOLD,
   *     with the threshold above / below every score, so every such row falls back
   *     (tests). */
  int32_t select_mode;
} lsa_semantic_params;

#define LSA_SEM_LIST_CAP 4096 /* entries of a decode row's threshold list */
enum {
  LSA_SEM_SELECT_ROW = 0,
  LSA_SEM_SELECT_THRESHOLD = 1,
  LSA_SEM_SELECT_FORCE_SHORT = 2,
  LSA_SEM_SELECT_FORCE_OVERFLOW = 3
};

/*
 * Bucket cache of blocks [first_block, first_block + n_update) of every sequence
 * ([LSA] §3.1 "Clustering", "Bucket cache"); the other blocks are left alone, so a
 * serving loop clusters each block once, when it completes.  k_idx: bf16
 * [B, L_max, 64]; (first_block + n_update) * n_cluster <= L_max; n_blocks: the
 * blocks the cache holds per sequence.  Layout (device memory, caller-owned):
 *   centroids bf16 [B, n_blocks, 8, 64, 8]: dims 8c..8c+7 of bucket s of a block at
 *     [c][s][0..7]; buckets of a block in order of the lowest pool key each holds
 *     (slots m..63 zero);
 *   table int32 [B, n_blocks, n_cluster]: the block's key positions (absolute within
 *     the sequence), bucket after bucket, ascending within a bucket;
 *   offsets int32 [B, n_blocks, m + 1]: bucket starts in table (offsets[m] = n_cluster).
 * Supported: d_idx = 64; n_cluster / n_pool <= 128 pool keys; m <= 64.  No workspace.
 */
lsa_status lsa_semantic_cluster(const void* k_idx, int32_t B, int32_t L_max, int32_t d_idx,
                                const lsa_semantic_params* prm, int32_t n_blocks, int32_t first_block,
                                int32_t n_update, void* centroids, int32_t* table, int32_t* offsets,
                                void* stream);

/*
 * Paged storage for the semantic search (serving layout; [LSA] App. F.1 "Flat decode": a
 * request's centroids lie in pages of the bucket cache and its keys in pages of the KV
 * cache, read through its page tables).  Either part may be NULL.
 *   block_table != NULL: the cache arrays of lsa_semantic_cluster/_select are pools of
 *     n_bslots entries (centroids bf16 [n_bslots, 8, 64, 8], table int32
 *     [n_bslots, n_cluster], offsets int32 [n_bslots, m + 1]) and block t of sequence b
 *     lives in entry block_table[b * n_blocks + t] (int32 [B, n_blocks]).  Table entries
 *     stay logical key positions.
 *   page_table != NULL: index keys (and, for the attention, K and V) are pools of n_slots
 *     rows, logical key j of sequence b at row page_table[b * max_pages + j / page_size]
 *     * page_size + j % page_size (page_size a power of two >= 64, L_max = max_pages *
 *     page_size, n_slots a multiple of page_size, at most 2^31); the index lists then hold
 *     those pool rows, in ascending logical order -- what lsa_sparse_attn reads from pools.
 * Ids outside their pools are clamped into them (no fault; the result is then
 * unspecified).
 */
typedef struct lsa_semantic_pages {
  const int32_t* block_table; /* int32 [B, n_blocks] or NULL */
  int32_t n_bslots;
  const int32_t* page_table;  /* int32 [B, max_pages] or NULL */
  int32_t page_size;
  int32_t max_pages;
  int64_t n_slots;
} lsa_semantic_pages;

/* lsa_semantic_cluster over paged storage (pages != NULL; see lsa_semantic_pages): with a
   page table, k_idx is the index-key pool bf16 [n_slots, 64] and L_max = max_pages *
   page_size. */
lsa_status lsa_semantic_cluster_paged(const void* k_idx, int32_t B, int32_t L_max, int32_t d_idx,
                                      const lsa_semantic_params* prm, const lsa_semantic_pages* pages,
                                      int32_t n_blocks, int32_t first_block, int32_t n_update, void* centroids,
                                      int32_t* table, int32_t* offsets, void* stream);

/* Workspace lsa_semantic_select needs to take all B * n_q queries in one pass: per
   query its normalised index query and one score-table row of n_blocks * m floats, and
   for decode (n_q == 1) rows of more than LSA_SEM_LIST_CAP buckets the threshold list
   (LSA_SEM_LIST_CAP 8-byte entries, a count and the threshold).  Less (at least one
   query per sequence) is accepted: the call then runs in chunks of queries. */
lsa_status lsa_semantic_select_workspace_size(int32_t B, int32_t n_q, int32_t n_blocks,
                                              const lsa_semantic_params* prm, size_t* bytes);

/*
 * Index lists of flat semantic search ([LSA] §3.2 "Scoring", "Expansion"): q_idx bf16
 * [B, n_q, 64]; q_pos int32 [B, n_q] (-1: padding query, empty list).  A query at p
 * scores the buckets of blocks 0 .. min(p / n_cluster, n_blocks) - 1 of the cache of
 * lsa_semantic_cluster (those blocks must be clustered), takes the top p_top and
 * expands them into at most k long-range keys.  idx int32 [B, n_q, n_sink + k + n_w]
 * receives the sink keys (j < min(n_sink, p + 1)), the long-range keys and the window
 * (max(0, p - n_w + 1) .. p), ascending and -1 padded; count int32 [B, n_q] their
 * number.  The list is that of the oracle bit for bit.  Attention over it:
 * lsa_sparse_attn with k_top = n_sink + k + n_w.
 * Supported: d_idx = 64; 1 <= k <= 4096; 1 <= p_top <= 2048.  ws 16-byte aligned.
 */
lsa_status lsa_semantic_select(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q, int32_t d_idx,
                               const lsa_semantic_params* prm, int32_t n_blocks, const void* centroids,
                               const int32_t* table, const int32_t* offsets, int32_t k, int32_t p_top,
                               int32_t n_sink, int32_t n_w, int32_t* idx, int32_t* count, void* ws,
                               size_t ws_bytes, void* stream);

/* lsa_semantic_select that also records three caller-created HIP events (hipEvent_t,
   passed as void*) on the stream: events[0] before the centroid scan of the last chunk of
   queries, events[1] after it, events[2] after the whole call -- how a benchmark times
   the scan and the selection live.  Same lists as lsa_semantic_select. */
lsa_status lsa_semantic_select_timed(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q,
                                     int32_t d_idx, const lsa_semantic_params* prm, int32_t n_blocks,
                                     const void* centroids, const int32_t* table, const int32_t* offsets, int32_t k,
                                     int32_t p_top, int32_t n_sink, int32_t n_w, int32_t* idx, int32_t* count,
                                     void* ws, size_t ws_bytes, void* stream, void* const* events);

/* lsa_semantic_select over paged storage (pages != NULL; see lsa_semantic_pages): the
   cache is read through the block table, and with a page table the lists hold pool rows
   (L_max = max_pages * page_size).  Same lists as the contiguous call, mapped. */
lsa_status lsa_semantic_select_paged(const void* q_idx, const int32_t* q_pos, int32_t B, int32_t n_q, int32_t d_idx,
                                     const lsa_semantic_params* prm, const lsa_semantic_pages* pages, int32_t L_max,
                                     int32_t n_blocks, const void* centroids, const int32_t* table,
                                     const int32_t* offsets, int32_t k, int32_t p_top, int32_t n_sink, int32_t n_w,
                                     int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
