"""The CPU oracle against its pins (no GPU).  See oracle_pins.py for what each pin is."""
from unittest import mock

import numpy as np
import pytest

from oracle import lsa_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes_pin(check):
    ok, msg = check(O)
    assert ok, msg


# ---------------------------------------------------------------- planted mistakes
# Each mutant is a plausible slip in the oracle.  Patched into the oracle module
# (so forward_row and friends use it too), it must fail at least one pin.

def _relu_after_sum(q_row, k_idx, w, p):
    n = min(int(p), k_idx.shape[0] - 1) + 1
    if n <= 0:
        return np.zeros((0,), np.int64)
    dots = O._int_dots(q_row, k_idx[:n])
    return np.maximum((np.asarray(w, np.int64)[:, None] * dots).sum(0), 0)


def _no_relu(q_row, k_idx, w, p):
    n = min(int(p), k_idx.shape[0] - 1) + 1
    if n <= 0:
        return np.zeros((0,), np.int64)
    dots = O._int_dots(q_row, k_idx[:n])
    return (np.asarray(w, np.int64)[:, None] * dots).sum(0)


def _exclusive_causal(q_row, k_idx, w, p):
    n = min(int(p), k_idx.shape[0])
    if n <= 0:
        return np.zeros((0,), np.int64)
    return O._weighted_relu_sum(O._int_dots(q_row, k_idx[:n]), w)


_orig_index_scores = O.index_scores
_orig_topk = O.topk
_orig_block_keep = O.block_keep
_orig_attn = O.sparse_attention


def _topk_high_index_ties(scores, cand, k):
    scores = np.asarray(scores, np.int64)
    cand = np.asarray(cand, np.int64)
    n = min(k, cand.shape[0])
    order = np.lexsort((-cand, -scores))
    J = np.full((k,), -1, np.int64)
    J[:n] = np.sort(cand[order[:n]])
    return J, n


def _topk_rank_order(scores, cand, k):
    scores = np.asarray(scores, np.int64)
    cand = np.asarray(cand, np.int64)
    n = min(k, cand.shape[0])
    order = np.lexsort((cand, -scores))
    J = np.full((k,), -1, np.int64)
    J[:n] = cand[order[:n]]
    return J, n


def _topk_smallest(scores, cand, k):
    return _orig_topk(-np.asarray(scores, np.int64), cand, k)


def _topk_off_by_one(scores, cand, k):
    J, n = _orig_topk(scores, cand, max(k - 1, 0))
    return np.concatenate([J, [-1]]), n


def _reps_mean(k_idx, block_size):
    k = np.asarray(k_idx, np.int64)
    n_blk = k.shape[0] // block_size
    return k[: n_blk * block_size].reshape(n_blk, block_size, k.shape[1]).sum(1) // block_size


def _reps_shifted(k_idx, block_size):
    k = np.asarray(k_idx, np.int64)[1:]
    n_blk = k.shape[0] // block_size
    return k[: n_blk * block_size].reshape(n_blk, block_size, k.shape[1]).sum(1)


def _keep_without_forcing_own(q_row, reps, w, p, block_size, n_keep):
    own = int(p) // block_size
    bs = O.block_scores(q_row, reps, w, own)
    m = np.arange(own)
    order = np.lexsort((m, -bs))
    best = m[order[: min(n_keep, own)]]
    kept = np.sort(np.concatenate([best, [own]]))
    return kept, bs


def _keep_high_index_ties(q_row, reps, w, p, block_size, n_keep):
    own = int(p) // block_size
    bs = O.block_scores(q_row, reps, w, own)
    m = np.arange(own)
    order = np.lexsort((-m, -bs))
    best = m[order[: min(n_keep - 1, own)]]
    return np.sort(np.concatenate([best, [own]])), bs


def _attn_wrong_scale(q_row, k_cache, v_cache, J, scale):
    return _orig_attn(q_row, k_cache, v_cache, J, 1.0 / scale)


def _attn_values_from_keys(q_row, k_cache, v_cache, J, scale):
    return _orig_attn(q_row, k_cache, k_cache, J, scale)


def _attn_padding_as_key(q_row, k_cache, v_cache, J, scale):
    J = np.asarray(J, np.int64)
    q = O._f64(q_row)
    Kj, Vj = O._f64(k_cache[J]), O._f64(v_cache[J])
    s = (q @ Kj.T) * scale
    m = s.max(1, keepdims=True)
    e = np.exp(s - m)
    return (e @ Vj) / e.sum(1, keepdims=True), (m + np.log(e.sum(1, keepdims=True)))[:, 0]


def _attn_lse_without_max(q_row, k_cache, v_cache, J, scale):
    out, lse = _orig_attn(q_row, k_cache, v_cache, J, scale)
    Jv = np.asarray(J)
    Jv = Jv[Jv >= 0]
    if Jv.size == 0:
        return out, lse
    m = ((O._f64(q_row) @ O._f64(k_cache[Jv]).T) * scale).max(1)
    return out, lse - m


def _cands_past_p(kept, p, block_size, L):
    keys = (np.asarray(kept, np.int64)[:, None] * block_size + np.arange(block_size)[None, :]).reshape(-1)
    return keys[keys < L]


_orig_paged_rows = O.paged_rows
_orig_forward_row_paged = O.forward_row_paged


def _paged_rows_no_offset(pt, n_keys, page_size):
    j = np.arange(n_keys, dtype=np.int64)
    return np.asarray(pt, np.int64)[j // page_size] * page_size


def _paged_rows_ignore_table(pt, n_keys, page_size):
    return np.arange(n_keys, dtype=np.int64)


def _paged_J_logical(*args, **kw):
    res = _orig_forward_row_paged(*args, **kw)
    res["J"] = res["J_logical"]
    return res


_orig_sem_ward_costs = O.sem_ward_costs
_orig_sem_ward = O.sem_ward
_orig_sem_expand = O.sem_expand


def _sem_cost_unweighted(S, cnt):
    S = np.asarray(S, np.float32)
    d = S[:, None, :] - S[None, :, :]
    return (d * d).sum(-1).astype(np.float32)


def _sem_cost_no_denominator(S, cnt):
    n = np.asarray(cnt).astype(np.float32)
    den = n[:, None] * n[None, :] * (n[:, None] + n[None, :])
    return (_orig_sem_ward_costs(S, cnt) * den).astype(np.float32)


def _no_trim(P, m, cap):
    # merges every mutual pair of the last round, so it may end below m buckets
    P = np.asarray(P, np.float32)
    n = P.shape[0]
    S, cnt, alive, lab, log = P.copy(), np.ones(n, np.int64), np.ones(n, bool), np.arange(n), []
    live, rnd = n, 0
    while live > m:
        C = O.sem_ward_costs(S, cnt)
        ok = alive[:, None] & alive[None, :] & ((cnt[:, None] + cnt[None, :]) <= cap)
        np.fill_diagonal(ok, False)
        partner = np.where(ok.any(1), np.argmin(np.where(ok, C, np.inf), axis=1), -1)
        pairs = [(a, int(partner[a])) for a in range(n) if alive[a] and partner[a] > a and partner[partner[a]] == a]
        if not pairs:
            break
        for a, b in pairs:
            log.append((rnd, a, b, float(C[a, b])))
            S[a] = S[a] + S[b]
            cnt[a] += cnt[b]
            alive[b] = False
            lab[lab == b] = a
        live -= len(pairs)
        rnd += 1
    return lab, S, cnt, log


def _sem_ward_greedy_nonmutual(P, m, cap):
    # every bucket merges with its partner whether or not the choice is mutual
    P = np.asarray(P, np.float32)
    n = P.shape[0]
    S, cnt, alive, lab, log = P.copy(), np.ones(n, np.int64), np.ones(n, bool), np.arange(n), []
    live, rnd = n, 0
    while live > m:
        C = O.sem_ward_costs(S, cnt)
        ok = alive[:, None] & alive[None, :] & ((cnt[:, None] + cnt[None, :]) <= cap)
        np.fill_diagonal(ok, False)
        if not ok.any():
            break
        a = int(np.nonzero(alive & ok.any(1))[0][0])
        b = int(np.argmin(np.where(ok[a], C[a], np.inf)))
        a, b = min(a, b), max(a, b)
        log.append((rnd, a, b, float(C[a, b])))
        S[a] = S[a] + S[b]
        cnt[a] += cnt[b]
        alive[b] = False
        lab[lab == b] = a
        live -= 1
        rnd += 1
    return lab, S, cnt, log


def _sem_expand_no_window_skip(best_first, table, offsets, p, k, n_sink, n_w):
    return _orig_sem_expand(best_first, table, offsets, p, k, n_sink, 0)


def _sem_top_high_ties(s, p_top):
    key = O.sem_order_key(s).astype(np.int64)
    order = np.lexsort((-np.arange(key.shape[0]), -key))
    return order[:p_top]


def _sem_pool_raw(k_blk, n_pool):
    y = np.asarray(k_blk, np.float32)
    n = y.shape[0] // n_pool
    return y[: n * n_pool].reshape(n, n_pool, -1).sum(1).astype(np.float32)


_orig_sem_scores = O.sem_scores


def _short(qn, cent):
    # the last index dimension left out of the dot product
    cent = np.asarray(cent, np.float32).copy()
    cent[:, -1] = 0
    return _orig_sem_scores(qn, cent)


def _sem_order_raw_bits(s):
    return np.asarray(s, np.float32).view(np.uint32).astype(np.uint64)


_orig_sem_cluster_block = O.sem_cluster_block


def _cluster_keys_descending(k_blk, n_pool, m, n_max, first_key=0):
    # each bucket's keys listed from the highest position down
    cent, table, off = _orig_sem_cluster_block(k_blk, n_pool, m, n_max, first_key)
    table = table.copy()
    for b in range(off.shape[0] - 1):
        table[off[b]:off[b + 1]] = table[off[b]:off[b + 1]][::-1]
    return cent, table, off


def _cluster_centroids_unrounded(k_blk, n_pool, m, n_max, first_key=0):
    # centroids left in fp32 instead of rounded to bf16
    _, table, off = _orig_sem_cluster_block(k_blk, n_pool, m, n_max, first_key)
    P = O.sem_pool_keys(k_blk, n_pool)
    lab, S, _, _ = O.sem_ward(P, m, n_max // n_pool)
    return O.sem_normalize(S[np.unique(lab)]), table, off


def _cluster_buckets_reversed(k_blk, n_pool, m, n_max, first_key=0):
    # a block's buckets listed in descending id order
    cent, table, off = _orig_sem_cluster_block(k_blk, n_pool, m, n_max, first_key)
    parts = [table[off[b]:off[b + 1]] for b in range(off.shape[0] - 1)][::-1]
    return cent[::-1].copy(), np.concatenate(parts), np.concatenate([[0], np.cumsum([len(x) for x in parts])])


MUTANTS = {
    "relu_after_sum": ("index_scores", _relu_after_sum),
    "no_relu": ("index_scores", _no_relu),
    "exclusive_causal": ("index_scores", _exclusive_causal),
    "weights_dropped": ("index_scores", lambda q, k, w, p: _orig_index_scores(q, k, np.ones_like(np.asarray(w)), p)),
    "topk_high_index_ties": ("topk", _topk_high_index_ties),
    "topk_rank_order": ("topk", _topk_rank_order),
    "topk_smallest": ("topk", _topk_smallest),
    "topk_off_by_one": ("topk", _topk_off_by_one),
    "reps_mean": ("block_reps", _reps_mean),
    "reps_shifted": ("block_reps", _reps_shifted),
    "keep_without_forcing_own": ("block_keep", _keep_without_forcing_own),
    "keep_high_index_ties": ("block_keep", _keep_high_index_ties),
    "attn_wrong_scale": ("sparse_attention", _attn_wrong_scale),
    "attn_values_from_keys": ("sparse_attention", _attn_values_from_keys),
    "attn_padding_as_key": ("sparse_attention", _attn_padding_as_key),
    "attn_lse_without_max": ("sparse_attention", _attn_lse_without_max),
    "cands_past_p": ("two_stage_candidates", _cands_past_p),
    "paged_rows_no_offset": ("paged_rows", _paged_rows_no_offset),
    "paged_rows_ignore_table": ("paged_rows", _paged_rows_ignore_table),
    "paged_J_logical": ("forward_row_paged", _paged_J_logical),
    "sem_cost_unweighted": ("sem_ward_costs", _sem_cost_unweighted),
    "sem_cost_no_denominator": ("sem_ward_costs", _sem_cost_no_denominator),
    "sem_ward_no_trim": ("sem_ward", _no_trim),
    "sem_ward_greedy_nonmutual": ("sem_ward", _sem_ward_greedy_nonmutual),
    "sem_expand_no_window_skip": ("sem_expand", _sem_expand_no_window_skip),
    "sem_top_high_ties": ("sem_top_buckets", _sem_top_high_ties),
    "sem_pool_raw_keys": ("sem_pool_keys", _sem_pool_raw),
    "sem_scores_last_dim_dropped": ("sem_scores", _short),
    "sem_order_raw_bits": ("sem_order_key", _sem_order_raw_bits),
    "sem_cluster_keys_descending": ("sem_cluster_block", _cluster_keys_descending),
    "sem_cluster_centroids_unrounded": ("sem_cluster_block", _cluster_centroids_unrounded),
    "sem_cluster_buckets_reversed": ("sem_cluster_block", _cluster_buckets_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    attr, fn = MUTANTS[name]
    failed = []
    with mock.patch.object(O, attr, fn):
        for check in P.ALL_CHECKS:
            try:
                ok, _ = check(O)
            except Exception:       # a crash also counts as caught
                ok = False
            if not ok:
                failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
