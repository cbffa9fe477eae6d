"""Plain CPU oracle of learned top-k sparse attention (numpy, one query row at a time).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Parity of every function
below is pinned by ``tests/test_oracle_pins.py`` (closed forms, invariants,
library routines, brute force); nothing here is "parity unpinned".

Sources (the pages this follows; all under the subject "learned sparse attention"):
  [LSA]  "Latent Sparse Attention (LSA)", paperpeel.com/paper/2610.42147:
         §2 "Sparse Attention" (cost model: O(Tk) prefill / O(k) decode),
         §2.1 "Design Choices", paragraph "Token Sparse Attention" (a cheap,
         narrow, low-precision scorer rates each earlier key; attention then
         uses only the chosen keys),
         §2.2 "Related Work" (two-stage block-then-token indexers),
         §3.1 "Semantic Clustering", paragraph "Pooling" (a pool key is the SUM
         of consecutive index keys),
         §3.2 "Semantic Search", paragraph "Attention" (one index list J_i is
         shared by all query heads),
         App. F.1 "Kernels", paragraph "Selection by threshold" (a 64-bit key
         ranks a higher score first and, at equal score, the lower id first;
         attention does not depend on the order of J_i),
         App. F.1, paragraph "Attention kernels" (J_i is a row of int32 slots
         padded with -1 when a query has fewer keys; attention reads the list as
         a page table -- with paged caches the slots are rows of the cache pool).
  [HISA] theflow.svmpsp.dev related-papers page, summary "HISA: Efficient
         Hierarchical Indexing for Fine-Grained Sparse Attention" (coarse block
         filter, then the original token indexer only inside kept blocks).
  [HyTopK] same page, summary of HyScale: HyTopK computes each query's EXACT
         top-k indices.

Readings where the pages are silent (each stated at its function):
  * score_j = sum_h w_h * max(0, q_h . k_j): the pages never print the token
    indexer's formula; this weighted-ReLU head sum in exact integers is the
    form the path is specified with.  One index key per token, shared by heads.
  * candidates of a query at position p are keys 0..p (the query's own key
    included), so |J| = min(k, p+1).
  * J is written in ascending key order and padded with -1.
  * attention: scale 1/sqrt(d), natural-base softmax, no extra mask.
  * paged caches: logical key j of a sequence is pool row
    page_table[j // page_size] * page_size + j % page_size; selection ranks
    logical keys (ties: lower logical index) and J holds the pool rows.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _int_dots(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact integer matrix a @ b.T through fp64 BLAS.

    Every product and partial sum of the int8 / block-sum operands used here is
    an integer of magnitude below 2^53, so the fp64 product is exact whatever
    the summation order, and rounding back to int64 recovers it.
    """
    return np.rint(_f64(a) @ _f64(b).T).astype(np.int64)


def _weighted_relu_sum(dots: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_h w_h * max(0, dots[h, :]) in int64 (ReLU per head, then weights)."""
    relu = np.maximum(dots, 0)
    return (np.asarray(w, dtype=np.int64)[:, None] * relu).sum(axis=0)


def index_scores(q_row, k_idx, w, p: int) -> np.ndarray:
    """Token-indexer scores of one query against keys 0..p (flat indexer).

    [LSA] §2.1 "Token Sparse Attention": the indexer scores every preceding key.
    q_row: int [H_I, d_I] (the query's index heads); k_idx: int [L, d_I] (one
    index key per token, shared by all heads); w: int [H_I]; p: position.
    Returns int64 [min(p, L-1) + 1]; empty for p < 0.
    """
    n = min(int(p), k_idx.shape[0] - 1) + 1
    if n <= 0:
        return np.zeros((0,), dtype=np.int64)
    dots = _int_dots(q_row, k_idx[:n])          # [H_I, n]
    return _weighted_relu_sum(dots, w)


def block_reps(k_idx, block_size: int) -> np.ndarray:
    """Representative of every complete key block: the int sum of its index keys.

    [LSA] §3.1 "Pooling" sums consecutive index keys into one; the two-stage
    indexer of [HISA] scores such block summaries.  Returns int64
    [L // block_size, d_I].
    """
    k = np.asarray(k_idx, dtype=np.int64)
    n_blk = k.shape[0] // block_size
    return k[: n_blk * block_size].reshape(n_blk, block_size, k.shape[1]).sum(axis=1)


def block_scores(q_row, reps, w, own: int) -> np.ndarray:
    """Block scores sum_h w_h * max(0, q_h . R_m) for the complete blocks m < own, int64."""
    if own <= 0:
        return np.zeros((0,), dtype=np.int64)
    dots = _int_dots(q_row, reps[:own])          # |q . R| <= 2^28: exact
    return _weighted_relu_sum(dots, w)


def block_keep(q_row, reps, w, p: int, block_size: int, n_keep: int):
    """Kept blocks of one query in the two-stage indexer ([HISA]; [LSA] §2.2).

    Reading: n_keep blocks in all -- the query's own (partial) block, always kept
    and never scored, plus the best n_keep-1 earlier blocks ranked by
    (block score descending, block index ascending).  With fewer than n_keep
    causal blocks every one is kept.  Returns (kept int64 ascending, scores).
    """
    own = int(p) // block_size
    bs = block_scores(q_row, reps, w, own)
    m = np.arange(own, dtype=np.int64)
    order = np.lexsort((m, -bs))                 # score desc, then index asc
    best = m[order[: min(n_keep - 1, own)]]
    kept = np.sort(np.concatenate([best, np.array([own], dtype=np.int64)]))
    return kept, bs


def two_stage_candidates(kept, p: int, block_size: int, L: int) -> np.ndarray:
    """Keys of the kept blocks that the query may see (j <= p), ascending."""
    keys = (np.asarray(kept, dtype=np.int64)[:, None] * block_size
            + np.arange(block_size, dtype=np.int64)[None, :]).reshape(-1)
    return keys[(keys <= p) & (keys < L)]


def topk(scores, cand, k: int):
    """Exact top-k of one row with lowest-index tie-break, ascending, -1 padded.

    [HyTopK] exact top-k; [LSA] App. F.1 "Selection by threshold": at equal score
    the lower id ranks first, and J's order does not matter to attention, so the
    canonical order here is ascending key index; "Attention kernels": rows are
    padded with -1.  Returns (J int64 [k], count = min(k, len(cand))).
    """
    scores = np.asarray(scores, dtype=np.int64)
    cand = np.asarray(cand, dtype=np.int64)
    n = min(k, cand.shape[0])
    order = np.lexsort((cand, -scores))
    sel = np.sort(cand[order[:n]])
    J = np.full((k,), -1, dtype=np.int64)
    J[:n] = sel
    return J, n


def sparse_attention(q_row, k_cache, v_cache, J, scale: float):
    """Softmax attention of one query's heads over the keys listed in J, in fp64.

    [LSA] §3.2 "Attention": attention over J_i only, one J_i for all heads;
    §2: this is the O(k)-per-query part.  q_row [H_q, d]; k_cache / v_cache
    [L, d]; J int [k] with -1 padding (ignored).  Returns (out [H_q, d] fp64,
    lse [H_q] fp64).  An empty J gives out = 0 and lse = -inf.
    """
    J = np.asarray(J, dtype=np.int64)
    J = J[J >= 0]
    q = _f64(q_row)
    if J.size == 0:
        return np.zeros_like(q), np.full((q.shape[0],), -np.inf)
    Kj = _f64(k_cache[J])
    Vj = _f64(v_cache[J])
    s = (q @ Kj.T) * scale                        # [H_q, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    out = (e @ Vj) / den
    lse = (m + np.log(den))[:, 0]
    return out, lse


def forward_row(q_idx_row, k_idx, w, p: int, k: int, q_row=None, k_cache=None,
                v_cache=None, scale: float | None = None, two_stage: bool = False,
                block_size: int = 128, n_keep: int = 64, reps=None, pooled: bool = False):
    """The whole path for one query row: candidates -> scores -> top-k -> attention.

    Flat: candidates are keys 0..p.  Two-stage ([HISA]): kept blocks first, then
    the same token scores over the kept keys.  Pooled (with two_stage; [LSA] §2.2
    "Related Work": indexers that score one pooled key per block of consecutive
    keys): the kept blocks' visible keys are the list itself, no token stage --
    J = those keys ascending, padded with -1 to k (k = n_keep * block_size).
    Returns a dict with J, count, and (if q_row is given) out / lse; the block modes
    add kept (padded to n_keep).
    """
    L = k_idx.shape[0]
    res = {}
    if two_stage:
        if reps is None:
            reps = block_reps(k_idx, block_size)
        kept, _ = block_keep(q_idx_row, reps, w, p, block_size, n_keep)
        cand = two_stage_candidates(kept, p, block_size, L)
        kp = np.full((n_keep,), -1, dtype=np.int64)
        kp[: kept.size] = kept
        res["kept"] = kp
        if pooled:
            J = np.full((k,), -1, dtype=np.int64)
            J[: cand.size] = cand
            res["J"], res["count"] = J, int(cand.size)
            if q_row is not None:
                if scale is None:
                    scale = 1.0 / np.sqrt(q_row.shape[-1])
                res["out"], res["lse"] = sparse_attention(q_row, k_cache, v_cache, J, scale)
            return res
        dots = _int_dots(q_idx_row, k_idx[cand]) if cand.size else np.zeros((len(w), 0), np.int64)
        sc = _weighted_relu_sum(dots, w)
    else:
        sc = index_scores(q_idx_row, k_idx, w, p)
        cand = np.arange(sc.shape[0], dtype=np.int64)
    J, cnt = topk(sc, cand, k)
    res["J"], res["count"] = J, cnt
    if q_row is not None:
        if scale is None:
            scale = 1.0 / np.sqrt(q_row.shape[-1])
        res["out"], res["lse"] = sparse_attention(q_row, k_cache, v_cache, J, scale)
    return res


def paged_rows(page_table_row, n_keys: int, page_size: int) -> np.ndarray:
    """Pool row of each logical key 0..n_keys-1 of one sequence with paged caches.

    [LSA] App. F.1 "Attention kernels": the index list is read like a page table.
    Reading: logical key j sits at offset j % page_size of the page named by
    entry j // page_size of the sequence's page table.
    """
    j = np.arange(n_keys, dtype=np.int64)
    pt = np.asarray(page_table_row, np.int64)
    return pt[j // page_size] * page_size + j % page_size


def forward_row_paged(q_idx_row, k_idx_pool, w, p: int, k: int, page_table_row, page_size: int,
                      q_row=None, k_pool=None, v_pool=None, scale: float | None = None):
    """The flat path for one query row of a sequence whose caches are paged.

    The sequence's logical caches are the pool rows its page table names
    (paged_rows); scores, top-k and attention are those of forward_row on them,
    and J then names the pool rows of the chosen logical keys (ascending logical
    order, -1 padded).  J_logical keeps the logical keys.
    """
    rows = paged_rows(page_table_row, len(page_table_row) * page_size, page_size)
    res = forward_row(q_idx_row, np.asarray(k_idx_pool)[rows], w, p, k, q_row=q_row,
                      k_cache=None if k_pool is None else np.asarray(k_pool)[rows],
                      v_cache=None if v_pool is None else np.asarray(v_pool)[rows], scale=scale)
    J = res["J"]
    res["J_logical"] = J
    res["J"] = np.where(J >= 0, rows[np.maximum(J, 0)], -1)
    return res
