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
                      q_row=None, k_pool=None, v_pool=None, scale: float | None = None, **modes):
    """The path for one query row of a sequence whose caches are paged.

    The sequence's logical caches are the pool rows its page table names
    (paged_rows); blocks, scores, top-k and attention are those of forward_row on
    them (``modes``: its two_stage / block_size / n_keep / pooled arguments, so blocks
    are blocks of logical keys and kept holds logical block ids), and J then names
    the pool rows of the chosen logical keys (ascending logical order, -1 padded).
    J_logical keeps the logical keys.
    """
    rows = paged_rows(page_table_row, len(page_table_row) * page_size, page_size)
    res = forward_row(q_idx_row, np.asarray(k_idx_pool)[rows], w, p, k, q_row=q_row,
                      k_cache=None if k_pool is None else np.asarray(k_pool)[rows],
                      v_cache=None if v_pool is None else np.asarray(v_pool)[rows], scale=scale, **modes)
    J = res["J"]
    res["J_logical"] = J
    res["J"] = np.where(J >= 0, rows[np.maximum(J, 0)], -1)
    return res


# =================================================================================
# Semantic search, flat ([LSA] §3.1 "Semantic Clustering", §3.2 "Semantic Search",
# App. F.1 "Kernels": "Selection by threshold", "Flat decode").
#
# Floating point decides integers here (which buckets merge, which are kept), so
# every such decision is taken in fp32 with each operation rounded on its own and
# sums over the index dimensions taken in order d = 0, 1, ...: the kernels follow
# the same definition and reach the same bits.  Readings where the pages are silent
# (listed again in the design notes):
#   * normalisation: ss = sum_d x_d * x_d, norm = sqrt(ss), x_d / norm, all fp32; a
#     zero vector stays zero;
#   * pool keys are sums of the *normalised* keys (normalisation comes first in §3.1),
#     summed in key order;
#   * Ward's cost of buckets a, b with sums S and sizes n (in pool keys):
#     |n_b S_a - n_a S_b|^2 / (n_a n_b (n_a + n_b)), the rise of the total squared
#     distance of the pool keys from their bucket means;
#   * a bucket's partner is its cheapest allowed merge, the lower id at equal cost;
#     ids are pool-key indices and a merged bucket keeps the lower id (so an id is
#     the lowest pool key a bucket holds);
#   * when merging every mutual pair of a round would leave fewer than m buckets,
#     only the cheapest pairs merge (cost, then lower id), so exactly m remain;
#   * centroids and index queries are normalised in fp32 and rounded to bf16 (the
#     pages score bf16 operands); a score is the fp32 sum of the exact products;
#   * a bucket's keys are listed in ascending position; buckets of a cluster block
#     by id.
# =================================================================================

_F32 = np.float32


def sem_bf16(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returned as fp32 values."""
    u = np.ascontiguousarray(x, dtype=_F32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(_F32)


def sem_normalize(x) -> np.ndarray:
    """L2 normalisation of every row in fp32 ([LSA] §3.1 "Key normalisation", §3.2
    "Query normalisation"): ss summed d = 0, 1, ..., each product and sum rounded;
    sqrt and division correctly rounded; a zero row stays zero."""
    x = np.asarray(x, _F32)
    ss = np.zeros(x.shape[:-1], _F32)
    for j in range(x.shape[-1]):
        ss = ss + x[..., j] * x[..., j]
    nrm = np.sqrt(ss)
    safe = np.where(nrm > 0, nrm, _F32(1)).astype(_F32)
    return np.where((nrm > 0)[..., None], x / safe[..., None], _F32(0)).astype(_F32)


def sem_pool_keys(k_blk, n_pool: int) -> np.ndarray:
    """Pool keys of a run of index keys ([LSA] §3.1 "Pooling"): every n_pool
    consecutive normalised keys summed, ((y0 + y1) + y2) + ..., in fp32."""
    y = sem_normalize(k_blk)
    n = y.shape[0] // n_pool
    y = y[: n * n_pool].reshape(n, n_pool, y.shape[-1])
    P = y[:, 0].copy()
    for i in range(1, n_pool):
        P = P + y[:, i]
    return P


def sem_ward_costs(S, cnt) -> np.ndarray:
    """Ward's merge cost of every pair of buckets ([LSA] §3.1 "Clustering", Ward's
    criterion): |n_b S_a - n_a S_b|^2 / (n_a n_b (n_a + n_b)) for bucket sums S [n, d]
    and sizes cnt [n] (pool keys), in fp32 with the squared norm summed d = 0, 1, ...
    Equal to n_a n_b / (n_a + n_b) * |mean_a - mean_b|^2, and symmetric bit for bit."""
    S = np.asarray(S, _F32)
    n = np.asarray(cnt).astype(_F32)
    na = n[:, None]
    nb = n[None, :]
    sq = np.zeros((S.shape[0], S.shape[0]), _F32)
    for j in range(S.shape[1]):
        dj = nb * S[:, None, j] - na * S[None, :, j]
        sq = sq + dj * dj
    return sq / (na * nb * (na + nb))


def sem_ward(P, m: int, cap: int):
    """Bottom-up Ward clustering of one cluster block's pool keys into m buckets
    ([LSA] §3.1 "Clustering").

    Every pool key starts as a bucket of its own (id = its index).  Each round, every
    bucket finds its cheapest allowed partner (a merge is allowed if the two hold at
    most ``cap`` pool keys together; lowest cost, then lowest id), and all pairs of
    buckets that are each other's partner merge at once; the merged bucket keeps the
    lower id and the sum of both sums.  If merging all of them would leave fewer than
    m buckets, only the cheapest pairs merge (cost, then lower id).  Stops at m
    buckets, or when no merge is allowed.

    Returns (label of every pool key = its bucket id, bucket sums [n, d] (rows of
    live ids), sizes [n], merge log [(round, a, b, cost)])."""
    P = np.asarray(P, _F32)
    n = P.shape[0]
    S = P.copy()
    cnt = np.ones(n, np.int64)
    alive = np.ones(n, bool)
    lab = np.arange(n)
    log = []
    live, rnd = n, 0
    while live > m:
        C = sem_ward_costs(S, cnt)
        ok = alive[:, None] & alive[None, :] & ((cnt[:, None] + cnt[None, :]) <= cap)
        np.fill_diagonal(ok, False)
        Cm = np.where(ok, C, np.inf)
        partner = np.where(ok.any(1), np.argmin(Cm, axis=1), -1)
        pairs = [(a, int(partner[a])) for a in range(n)
                 if alive[a] and partner[a] > a and partner[partner[a]] == a]
        if not pairs:
            break
        if live - len(pairs) < m:
            pairs.sort(key=lambda ab: (C[ab[0], ab[1]], ab[0]))
            pairs = pairs[: live - m]
        for a, b in pairs:
            log.append((rnd, a, b, float(C[a, b])))
            S[a] = S[a] + S[b]
            cnt[a] += cnt[b]
            alive[b] = False
            lab[lab == b] = a
        live -= len(pairs)
        rnd += 1
    return lab, S, cnt, log


def sem_cluster_block(k_blk, n_pool: int, m: int, n_max: int, first_key: int = 0):
    """One complete cluster block into its bucket-cache entry ([LSA] §3.1 "Clustering",
    "Bucket cache").  k_blk: the block's n_cluster index keys [n_cluster, d] (bf16
    values).  Returns (centroids [n_b, d]: each bucket's sum normalised and rounded to
    bf16; table [n_cluster]: key positions, bucket after bucket in id order, each
    bucket's keys ascending; offsets [n_b + 1] into the table).  n_b = m unless the
    size cap stopped the merging early."""
    P = sem_pool_keys(k_blk, n_pool)
    lab, S, _, _ = sem_ward(P, m, n_max // n_pool)
    ids = np.unique(lab)
    cent = sem_bf16(sem_normalize(S[ids]))
    table, off = [], [0]
    for b in ids:
        for u in np.nonzero(lab == b)[0]:
            table.extend(range(first_key + int(u) * n_pool, first_key + (int(u) + 1) * n_pool))
        off.append(len(table))
    return cent, np.asarray(table, np.int64), np.asarray(off, np.int64)


def bucket_cache(k_idx, n_cluster: int, n_pool: int, n_bavg: int, n_max: int, n_blocks=None) -> dict:
    """Bucket cache of one sequence ([LSA] §3.1 "Bucket cache"): every complete cluster
    block of k_idx [L, d] (or the first n_blocks) clustered into m = n_cluster / n_bavg
    buckets.  Returns dict(centroids [NB, m, d], table [NB, n_cluster], offsets
    [NB, m + 1], n_cluster)."""
    k_idx = np.asarray(k_idx, _F32)
    m = n_cluster // n_bavg
    nb = k_idx.shape[0] // n_cluster if n_blocks is None else n_blocks
    cents, tabs, offs = [], [], []
    for blk in range(nb):
        c, t, o = sem_cluster_block(k_idx[blk * n_cluster:(blk + 1) * n_cluster], n_pool, m, n_max,
                                    first_key=blk * n_cluster)
        assert c.shape[0] == m, "size cap left more than m buckets"
        cents.append(c)
        tabs.append(t)
        offs.append(o)
    d = k_idx.shape[1]
    return {"centroids": np.asarray(cents, _F32).reshape(nb, m, d),
            "table": np.asarray(tabs, np.int64).reshape(nb, n_cluster),
            "offsets": np.asarray(offs, np.int64).reshape(nb, m + 1), "n_cluster": n_cluster}


def sem_scores(qn, cent) -> np.ndarray:
    """s_b = c_b . q for every bucket ([LSA] §3.2 "Scoring"): bf16 operands, every
    product exact in fp32, the sum taken d = 0, 1, ... with each addition rounded."""
    qn = np.asarray(qn, _F32)
    cent = np.asarray(cent, _F32)
    s = np.zeros(cent.shape[0], _F32)
    for j in range(cent.shape[1]):
        s = s + cent[:, j] * qn[j]
    return s


def sem_order_key(s) -> np.ndarray:
    """Order-keeping unsigned image of fp32 scores (the upper half of the packed key of
    [LSA] App. F.1 "Selection by threshold"): a higher score gives a larger key; -0
    sits just below +0."""
    u = np.asarray(s, _F32).view(np.uint32).astype(np.uint64)
    return np.where((u >> 31) == 1, u ^ 0xFFFFFFFF, u | 0x80000000)


def sem_top_buckets(s, p_top: int) -> np.ndarray:
    """The top-p buckets of a row, best first: the larger packed key first, i.e. the
    higher score, at equal keys the lower bucket id ([LSA] §3.2 "Scoring",
    App. F.1 "Selection by threshold")."""
    key = sem_order_key(s).astype(np.int64)
    order = np.lexsort((np.arange(key.shape[0]), -key))
    return order[:p_top]


def sem_expand(best_first, table, offsets, p: int, k: int, n_sink: int, n_w: int) -> np.ndarray:
    """Long-range keys of one query ([LSA] §3.2 "Expansion"): the selected buckets best
    first, each bucket's keys in table order, skipping keys of the sink (j < n_sink) and
    of the window (j > p - n_w), until k keys."""
    m = offsets.shape[1] - 1
    w0 = max(0, p - n_w + 1)
    out = []
    for b in best_first:
        if len(out) >= k:
            break
        blk, loc = divmod(int(b), m)
        for j in table[blk, offsets[blk, loc]:offsets[blk, loc + 1]]:
            if j < n_sink or j >= w0:
                continue
            out.append(int(j))
            if len(out) == k:
                break
    return np.asarray(out, np.int64)


def semantic_select_row(q_idx_row, cache: dict, p: int, k: int, p_top: int, n_sink: int, n_w: int) -> dict:
    """Index list J_i of one query under flat semantic search ([LSA] §3.2): the query
    (normalised, bf16) scores every bucket of the cluster blocks before its own, keeps
    the top-p, expands them into k long-range keys; J_i adds the sink keys and the
    window (p - n_w, p].  Ascending, -1 padded to n_sink + k + n_w.
    Returns dict(J, count, kept (best first), scores)."""
    width = n_sink + k + n_w
    J = np.full((width,), -1, np.int64)
    if p < 0:
        return {"J": J, "count": 0, "kept": np.zeros(0, np.int64), "scores": np.zeros(0, _F32)}
    n_c = cache["n_cluster"]
    cent = cache["centroids"]
    m = cent.shape[1]
    nb = p // n_c
    assert nb <= cent.shape[0], "bucket cache lacks blocks before the query's own"
    qn = sem_bf16(sem_normalize(np.asarray(q_idx_row, _F32)))
    s = sem_scores(qn, cent[:nb].reshape(nb * m, cent.shape[2]))
    kept = sem_top_buckets(s, p_top)
    lr = sem_expand(kept, cache["table"], cache["offsets"], p, k, n_sink, n_w)
    w0 = max(0, p - n_w + 1)
    keys = sorted(set(range(min(n_sink, p + 1))) | set(range(w0, p + 1)) | set(lr.tolist()))
    J[:len(keys)] = keys
    return {"J": J, "count": len(keys), "kept": kept, "scores": s}


def semantic_forward_row(q_idx_row, cache: dict, p: int, k: int, p_top: int, n_sink: int, n_w: int,
                         q_row=None, k_cache=None, v_cache=None, scale: float | None = None) -> dict:
    """Flat semantic search for one query, then attention over J_i ([LSA] §3.2
    "Attention": one J_i for all heads)."""
    r = semantic_select_row(q_idx_row, cache, p, k, p_top, n_sink, n_w)
    if q_row is not None:
        if scale is None:
            scale = 1.0 / np.sqrt(np.asarray(q_row).shape[-1])
        r["out"], r["lse"] = sparse_attention(q_row, k_cache, v_cache, r["J"], scale)
    return r
