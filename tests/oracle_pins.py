"""Pins of the CPU oracle: checks that do not re-derive the oracle's own code.

Each ``check_*`` takes the implementation under test as an argument and returns
``(ok, message)``.  ``test_oracle_pins.py`` runs them on the real oracle (all
must pass) and on planted mistakes of it (each mutant must fail at least one),
which shows that a plausible slip in the oracle -- a dropped term, a wrong sign
or index, ReLU in the wrong place, the wrong tie-break -- would not go unseen.

Kinds of pin used (nothing here calls the oracle to produce its own expected
values):
  * hand-worked examples (tests/golden/hand_worked.json);
  * closed forms of special inputs (one head / one dim; constant vectors);
  * invariances the definition implies (head / dim permutation, linearity in w);
  * brute force by a different route (rank counting instead of sorting);
  * library routines (torch scaled_dot_product_attention in fp64, scipy logsumexp);
  * reductions of the two-stage indexer to the flat one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _ok(cond, msg):
    return (bool(cond), msg)


def _all(results):
    for ok, msg in results:
        if not ok:
            return False, msg
    return True, "ok"


# ----------------------------------------------------------------------------- scores
def check_scores_hand(impl):
    g = _load_golden()["indexer"]
    q, w, K = np.array(g["q"]), np.array(g["w"]), np.array(g["k_idx"])
    r = []
    r.append(_ok(np.array_equal(impl.index_scores(q, K, w, 5), g["scores_p5"]), "hand scores p=5"))
    r.append(_ok(np.array_equal(impl.index_scores(q, K, w, 3), g["scores_p3"]), "hand scores p=3"))
    return _all(r)


def check_scores_closed_forms(impl, seed=0):
    rng = np.random.default_rng(seed)
    r = []
    # one head, one dim, unit weight: S_j = max(0, q * k_j)
    for _ in range(5):
        L = int(rng.integers(1, 40))
        q = rng.integers(-64, 65, size=(1, 1))
        K = rng.integers(-64, 65, size=(L, 1))
        p = int(rng.integers(0, L))
        want = [max(0, int(q[0, 0]) * int(K[j, 0])) for j in range(p + 1)]
        r.append(_ok(np.array_equal(impl.index_scores(q, K, np.array([1]), p), want), "H=d=1 closed form"))
    # q = +1 everywhere, k_j = c_j * ones: S_j = d * max(0, c_j) * sum(w)
    for H, d in ((3, 5), (4, 64), (64, 128)):
        w = rng.integers(1, 17, size=H)
        c = rng.integers(-64, 65, size=50)
        K = np.repeat(c[:, None], d, axis=1)
        q = np.ones((H, d), dtype=np.int64)
        want = [d * max(0, int(cj)) * int(w.sum()) for cj in c]
        r.append(_ok(np.array_equal(impl.index_scores(q, K, w, 49), want), f"constant vectors H={H} d={d}"))
    return _all(r)


def check_scores_invariances(impl, seed=1):
    rng = np.random.default_rng(seed)
    H, d, L = 8, 16, 60
    q = rng.integers(-64, 65, size=(H, d))
    K = rng.integers(-64, 65, size=(L, d))
    w = rng.integers(1, 17, size=H)
    p = L - 1
    s = impl.index_scores(q, K, w, p)
    r = []
    ph = rng.permutation(H)
    r.append(_ok(np.array_equal(impl.index_scores(q[ph], K, w[ph], p), s), "head permutation"))
    pd = rng.permutation(d)
    r.append(_ok(np.array_equal(impl.index_scores(q[:, pd], K[:, pd], w, p), s), "dim permutation"))
    r.append(_ok(np.array_equal(impl.index_scores(-q, -K, w, p), s), "joint negation"))
    w2 = rng.integers(1, 17, size=H)
    s2 = impl.index_scores(q, K, w2, p)
    r.append(_ok(np.array_equal(impl.index_scores(q, K, w + w2, p), s + s2), "additive in w"))
    r.append(_ok(np.array_equal(impl.index_scores(q, K, 3 * w, p), 3 * s), "homogeneous in w"))
    # one head alone: S = w * max(0, dot) where dot = sum of elementwise products
    for h in range(H):
        e = np.zeros(H, dtype=np.int64)
        e[h] = 1
        dots = [sum(int(q[h, t]) * int(K[j, t]) for t in range(d)) for j in range(L)]
        r.append(_ok(np.array_equal(impl.index_scores(q, K, e, p), [max(0, x) for x in dots]), f"single head {h}"))
    # causality: p+1 keys, prefix-consistent, p clipped to the cache, p < 0 empty
    r.append(_ok(len(impl.index_scores(q, K, w, 10)) == 11, "length p+1"))
    r.append(_ok(np.array_equal(impl.index_scores(q, K, w, 10), s[:11]), "prefix consistency"))
    r.append(_ok(len(impl.index_scores(q, K, w, L + 5)) == L, "p clipped to L-1"))
    r.append(_ok(len(impl.index_scores(q, K, w, -1)) == 0, "p<0 empty"))
    return _all(r)


def check_scores_bound(impl, seed=2):
    """Extreme inputs of the workloads' ranges stay below 2^31 (int32 scores are exact)."""
    H, d = 64, 128
    q = np.full((H, d), 64)
    K = np.full((4, d), 64)
    w = np.full(H, 16)
    s = impl.index_scores(q, K, w, 3)
    want = H * 16 * d * 64 * 64
    return _all([_ok(np.all(s == want), "extreme score value"), _ok(want < 2 ** 31, "int32 bound")])


# ----------------------------------------------------------------------------- top-k
def _bruteforce_topk(scores, cand, k):
    """Selected iff fewer than k candidates beat it (higher score, or equal score and lower index)."""
    sel = []
    n = len(cand)
    for a in range(n):
        beat = 0
        for b in range(n):
            if scores[b] > scores[a] or (scores[b] == scores[a] and cand[b] < cand[a]):
                beat += 1
        if beat < k:
            sel.append(int(cand[a]))
    sel.sort()
    return sel + [-1] * (k - len(sel))


def check_topk_hand(impl):
    g = _load_golden()["indexer"]
    s5 = np.array(g["scores_p5"])
    r = []
    for c in g["topk_cases"]:
        s = s5[: c["p"] + 1]
        J, cnt = impl.topk(s, np.arange(c["p"] + 1), c["k"])
        r.append(_ok(list(J) == c["J"] and cnt == c["count"], f"hand top-k p={c['p']} k={c['k']}"))
    return _all(r)


def check_topk_bruteforce(impl, seed=3):
    rng = np.random.default_rng(seed)
    r = []
    for trial in range(40):
        n = int(rng.integers(1, 200))
        hi = int(rng.choice([1, 2, 5, 1000, 2 ** 30]))
        scores = rng.integers(-hi, hi + 1, size=n)
        cand = np.sort(rng.choice(4 * n + 10, size=n, replace=False))
        for k in sorted({1, 7, 64, n, max(1, n // 2)}):
            J, cnt = impl.topk(scores, cand, k)
            r.append(_ok(list(J) == _bruteforce_topk(scores, cand, k) and cnt == min(k, n),
                         f"brute force n={n} k={k} trial={trial}"))
    return _all(r)


def check_topk_special(impl):
    r = []
    n = 100
    ar = np.arange(n)
    J, _ = impl.topk(np.zeros(n, dtype=np.int64), ar, 10)
    r.append(_ok(list(J) == list(range(10)), "all equal -> lowest indices"))
    J, _ = impl.topk(ar.copy(), ar, 10)
    r.append(_ok(list(J) == list(range(n - 10, n)), "increasing -> last k"))
    J, _ = impl.topk(-ar, ar, 10)
    r.append(_ok(list(J) == list(range(10)), "decreasing -> first k"))
    J, cnt = impl.topk(ar[:5], ar[:5], 8)
    r.append(_ok(list(J) == [0, 1, 2, 3, 4, -1, -1, -1] and cnt == 5, "t < k pads with -1"))
    J, cnt = impl.topk(np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64), 3)
    r.append(_ok(list(J) == [-1, -1, -1] and cnt == 0, "empty row"))
    s = np.array([1, 0, 1, 0, 1, -1, 0, 1])
    J, _ = impl.topk(s, np.arange(8), 5)
    r.append(_ok(list(J) == [0, 1, 2, 4, 7], "{-1,0,1} ties"))
    return _all(r)


# ----------------------------------------------------------------------------- blocks
def check_blocks_hand(impl):
    g = _load_golden()
    gi, gt = g["indexer"], g["two_stage"]
    q, w, K = np.array(gi["q"]), np.array(gi["w"]), np.array(gi["k_idx"])
    bs = gt["block_size"]
    r = [_ok(np.array_equal(impl.block_reps(K, bs), gt["reps"]), "hand reps")]
    reps = impl.block_reps(K, bs)
    r.append(_ok(np.array_equal(impl.block_scores(q, reps, w, 2), gt["block_scores_p5"]), "hand block scores"))
    for c in gt["cases"]:
        kept, _ = impl.block_keep(q, reps, w, c["p"], bs, c["n_keep"])
        res = impl.forward_row(q, K, w, c["p"], c["k"], two_stage=True, block_size=bs, n_keep=c["n_keep"])
        r.append(_ok(list(kept) == c["kept"], f"hand kept p={c['p']} n_keep={c['n_keep']}"))
        r.append(_ok(list(res["J"]) == c["J"], f"hand two-stage J p={c['p']} k={c['k']}"))
    return _all(r)


def check_block_reps_sum(impl, seed=4):
    rng = np.random.default_rng(seed)
    K = rng.integers(-64, 65, size=(16 * 7 + 5, 6))
    R = impl.block_reps(K, 16)
    r = [_ok(R.shape == (7, 6), "complete blocks only")]
    for m in range(7):
        want = [sum(int(K[16 * m + t, c]) for t in range(16)) for c in range(6)]
        r.append(_ok(list(R[m]) == want, f"block {m} sum"))
    return _all(r)


def check_block_keep_bruteforce(impl, seed=5):
    """Kept set = own + blocks that fewer than n_keep-1 earlier blocks beat."""
    rng = np.random.default_rng(seed)
    r = []
    for trial in range(12):
        T, bs, n_keep, H, d = 512, 16, 4, 3, 8
        K = rng.integers(-2, 3, size=(T, d))           # narrow range: many ties
        q = rng.integers(-2, 3, size=(H, d))
        w = rng.integers(1, 4, size=H)
        R = impl.block_reps(K, bs)
        for p in (0, 15, 16, 47, 63, 64, 200, 511):
            own = p // bs
            bsc = []
            for m in range(own):
                tot = 0
                for h in range(H):
                    dot = sum(int(q[h, t]) * int(R[m, t]) for t in range(d))
                    tot += int(w[h]) * max(0, dot)
                bsc.append(tot)
            want = [own]
            for m in range(own):
                beat = sum(1 for m2 in range(own) if bsc[m2] > bsc[m] or (bsc[m2] == bsc[m] and m2 < m))
                if beat < n_keep - 1:
                    want.append(m)
            kept, _ = impl.block_keep(q, R, w, p, bs, n_keep)
            r.append(_ok(list(kept) == sorted(want), f"block keep brute force p={p} trial={trial}"))
    return _all(r)


def check_two_stage_reductions(impl, seed=6):
    rng = np.random.default_rng(seed)
    r = []
    H, d, T = 4, 16, 300
    K = rng.integers(-64, 65, size=(T, d))
    w = rng.integers(1, 17, size=H)
    for p in (0, 5, 63, 127, 255, 299):
        q = rng.integers(-64, 65, size=(H, d))
        flat = impl.forward_row(q, K, w, p, 24)["J"]
        # 1) every causal block kept (own < n_keep): two-stage equals flat
        two = impl.forward_row(q, K, w, p, 24, two_stage=True, block_size=16, n_keep=T // 16 + 1)["J"]
        r.append(_ok(np.array_equal(flat, two), f"all blocks kept p={p}"))
        # 2) block size 1 and n_keep >= k+1: two-stage equals flat
        two1 = impl.forward_row(q, K, w, p, 24, two_stage=True, block_size=1, n_keep=25)["J"]
        r.append(_ok(np.array_equal(flat, two1), f"block size 1 p={p}"))
    return _all(r)


def check_two_stage_invariants(impl, seed=7):
    rng = np.random.default_rng(seed)
    H, d, T, bs, n_keep = 4, 16, 2048, 16, 8
    K = rng.integers(-64, 65, size=(T, d))
    w = rng.integers(1, 17, size=H)
    R = impl.block_reps(K, bs)
    r = []
    for p in (3, 16 * 5, 16 * 7 + 3, 16 * 8, 1000, 2047):
        q = rng.integers(-64, 65, size=(H, d))
        kept, _ = impl.block_keep(q, R, w, p, bs, n_keep)
        own = p // bs
        r.append(_ok(len(kept) == min(n_keep, own + 1), f"kept count p={p}"))
        r.append(_ok(own in set(kept.tolist()), f"own kept p={p}"))
        r.append(_ok(np.all(np.diff(kept) > 0), f"kept ascending p={p}"))
    return _all(r)


# ----------------------------------------------------------------------------- attention
def check_attention_hand(impl):
    g = _load_golden()["attention"]
    r = []
    for name in ("case_weighted", "case_zero_query"):
        c = g[name]
        q, k, v = np.array(c["q"]), np.array(c["k"]), np.array(c["v"])
        out, lse = impl.sparse_attention(q, k, v, np.array(c["J"]), 1.0 / math.sqrt(2.0))
        r.append(_ok(np.allclose(out, c["out"], atol=1e-12, rtol=0), f"hand attention {name} out"))
        r.append(_ok(np.allclose(lse, c["lse"], atol=1e-12, rtol=0), f"hand attention {name} lse"))
    return _all(r)


def check_attention_dense(impl, seed=8):
    """k >= t+1: sparse attention over all causal keys equals dense causal attention (torch SDPA, fp64)."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp
    rng = np.random.default_rng(seed)
    T, H, d = 40, 4, 16
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    scale = 1.0 / math.sqrt(d)
    tq = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)         # [1, H, T, d]
    tk = torch.from_numpy(k)[None, None].expand(1, H, T, d)
    tv = torch.from_numpy(v)[None, None].expand(1, H, T, d)
    dense = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)[0].permute(1, 0, 2).numpy()
    r = []
    for t in range(T):
        J = np.concatenate([np.arange(t + 1), -np.ones(T + 3 - (t + 1), dtype=np.int64)])
        out, lse = impl.sparse_attention(q[t], k, v, J, scale)
        r.append(_ok(np.max(np.abs(out - dense[t])) < 1e-12, f"dense equality t={t}"))
        want_lse = logsumexp((q[t] @ k[: t + 1].T) * scale, axis=1)
        r.append(_ok(np.max(np.abs(lse - want_lse)) < 1e-12, f"lse t={t}"))
    return _all(r)


def check_attention_special(impl, seed=9):
    rng = np.random.default_rng(seed)
    H, d, L = 4, 32, 50
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    scale = 1.0 / math.sqrt(d)
    r = []
    out, _ = impl.sparse_attention(q, k, v, np.array([7, -1, -1]), scale)
    r.append(_ok(np.array_equal(out, np.repeat(v[7][None], H, 0)), "single key -> V[j]"))
    J = np.array([1, 4, 9, 20, 33, -1])
    out, _ = impl.sparse_attention(np.zeros((H, d)), k, v, J, scale)
    r.append(_ok(np.allclose(out, np.repeat(v[[1, 4, 9, 20, 33]].mean(0)[None], H, 0), atol=1e-14), "zero query -> mean"))
    out1, lse1 = impl.sparse_attention(q, k, v, J, scale)
    out2, lse2 = impl.sparse_attention(q, k, v, J[[3, 0, 5, 2, 4, 1]], scale)
    r.append(_ok(np.allclose(out1, out2, atol=1e-14) and np.allclose(lse1, lse2, atol=1e-14), "permutation invariance"))
    qq = np.repeat(q[:1], H, 0)
    out, _ = impl.sparse_attention(qq, k, v, J, scale)
    r.append(_ok(all(np.array_equal(out[0], out[h]) for h in range(H)), "identical heads"))
    # split-and-merge by log-sum-exp equals the whole (the decode split combine)
    Ja, Jb = J[:2], J[2:5]
    oa, la = impl.sparse_attention(q, k, v, Ja, scale)
    ob, lb = impl.sparse_attention(q, k, v, Jb, scale)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (oa * wa[:, None] + ob * wb[:, None]) / (wa + wb)[:, None]
    r.append(_ok(np.allclose(merged, out1, atol=1e-13), "LSE split merge"))
    r.append(_ok(np.allclose(m + np.log(wa + wb), lse1, atol=1e-13), "LSE merge of lse"))
    out, lse = impl.sparse_attention(q, k, v, np.array([-1, -1]), scale)
    r.append(_ok(np.all(out == 0) and np.all(np.isneginf(lse)), "empty list -> zeros, -inf"))
    # a sharp query: attention goes to the argmax key
    J2 = np.array([3, 8, 13])
    qs = np.repeat((k[8] * 200.0)[None], H, 0)
    out, _ = impl.sparse_attention(qs, k, v, J2, scale)
    r.append(_ok(np.allclose(out, np.repeat(v[8][None], H, 0), atol=1e-9), "sharp query -> argmax key"))
    return _all(r)


def check_pooled_hand(impl):
    """Pooled blocks by hand: one head, one dim, w = 1, q = 1, so a block's score is
    max(0, the sum of its keys)."""
    k_idx = np.array([[3], [1], [0], [5], [2], [2], [4], [0], [1], [1]], np.int64)
    q = np.array([[1]], np.int64)
    w = np.array([1], np.int64)
    r = []
    # blocks of 2: sums 4 5 4 4 2.  p = 8: own block 4 (keys 8, 9; only 8 visible); the best
    # two earlier blocks are 1 (5) and, among the ties at 4, block 0
    res = impl.forward_row(q, k_idx, w, 8, 6, two_stage=True, block_size=2, n_keep=3, pooled=True)
    r.append(_ok(np.array_equal(res["J"], [0, 1, 2, 3, 8, -1]) and res["count"] == 5
                 and np.array_equal(res["kept"], [0, 1, 4]), f"p=8 {res['J']}"))
    res = impl.forward_row(q, k_idx, w, 9, 6, two_stage=True, block_size=2, n_keep=3, pooled=True)
    r.append(_ok(np.array_equal(res["J"], [0, 1, 2, 3, 8, 9]) and res["count"] == 6, f"p=9 {res['J']}"))
    res = impl.forward_row(q, k_idx, w, 1, 6, two_stage=True, block_size=2, n_keep=3, pooled=True)
    r.append(_ok(np.array_equal(res["J"], [0, 1, -1, -1, -1, -1]) and res["count"] == 2, f"p=1 {res['J']}"))
    # a negative query: every block score is ReLU'd to 0, ties go to the lowest blocks
    res = impl.forward_row(-q, k_idx, w, 7, 6, two_stage=True, block_size=2, n_keep=3, pooled=True)
    r.append(_ok(np.array_equal(res["J"], [0, 1, 2, 3, 6, 7]), f"all ties {res['J']}"))
    return _all(r)


def check_pooled_dense(impl, seed=12):
    """Enough kept blocks for every block up to the query's: the list is every key
    0..p (the flat list with k > p), and attention is dense causal attention."""
    rng = np.random.default_rng(seed)
    L, d_I, d, H, bs = 40, 16, 8, 3, 4
    k_idx = rng.integers(-64, 65, (L, d_I))
    kc, vc = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    q_idx = rng.integers(-64, 65, (H, d_I))
    w = rng.integers(1, 17, (H,))
    q = rng.standard_normal((H, d))
    r = []
    for p in (0, 5, 17, 39):
        res = impl.forward_row(q_idx, k_idx, w, p, 40, q_row=q, k_cache=kc, v_cache=vc, two_stage=True,
                               block_size=bs, n_keep=10, pooled=True)
        want = np.concatenate([np.arange(p + 1), np.full(40 - p - 1, -1)])
        s = (q @ kc[: p + 1].T) / math.sqrt(d)
        e = np.exp(s - s.max(1, keepdims=True))
        dense = (e @ vc[: p + 1]) / e.sum(1, keepdims=True)
        r.append(_ok(np.array_equal(res["J"], want) and res["count"] == p + 1
                     and np.allclose(res["out"], dense, atol=1e-13), f"dense p={p}"))
    return _all(r)


def check_paged_hand(impl):
    """Paged caches by hand: pool rows of logical keys, and one worked selection."""
    r = []
    r.append(_ok(np.array_equal(impl.paged_rows([2, 0, 1], 6, 2), [4, 5, 0, 1, 2, 3]), "rows, pages of 2"))
    r.append(_ok(np.array_equal(impl.paged_rows([3, 1], 8, 4), [12, 13, 14, 15, 4, 5, 6, 7]), "rows, pages of 4"))
    # one head, one dim, w = 1, q = 1: a key's score is max(0, its value).  Pool rows hold
    # 5 1 7 3 2 9; the page table [1, 2, 0] makes the logical keys 7 3 2 9 5 1.
    pool = np.array([[5], [1], [7], [3], [2], [9]], np.int64)
    q = np.array([[1]], np.int64)
    w = np.array([1], np.int64)
    res = impl.forward_row_paged(q, pool, w, 5, 3, [1, 2, 0], 2)
    # best three logical keys: 3 (9), 0 (7), 4 (5) -> logical [0, 3, 4] -> pool rows [2, 5, 0]
    r.append(_ok(np.array_equal(res["J"], [2, 5, 0]) and res["count"] == 3, f"worked selection {res['J']}"))
    res = impl.forward_row_paged(q, pool, w, 3, 2, [1, 2, 0], 2)
    r.append(_ok(np.array_equal(res["J"], [2, 5]), f"causal limit {res['J']}"))
    res = impl.forward_row_paged(q, pool, w, 1, 4, [1, 2, 0], 2)
    r.append(_ok(np.array_equal(res["J"], [2, 3, -1, -1]), f"short row padded {res['J']}"))
    return _all(r)


def _paged_case(rng, n_pages_seq, page_size, spare, d_I=16, d=8, H=4):
    L = n_pages_seq * page_size
    k_idx = rng.integers(-64, 65, (L, d_I))
    kc = rng.standard_normal((L, d))
    vc = rng.standard_normal((L, d))
    n_pool = n_pages_seq + spare
    perm = rng.permutation(n_pool)[:n_pages_seq]
    rows = (perm[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)
    pool_k_idx = rng.integers(-64, 65, (n_pool * page_size, d_I))
    pool_kc = rng.standard_normal((n_pool * page_size, d))
    pool_vc = rng.standard_normal((n_pool * page_size, d))
    pool_k_idx[rows], pool_kc[rows], pool_vc[rows] = k_idx, kc, vc
    q_idx = rng.integers(-64, 65, (H, d_I))
    w = rng.integers(1, 17, (H,))
    q = rng.standard_normal((H, d))
    return L, k_idx, kc, vc, perm, pool_k_idx, pool_kc, pool_vc, q_idx, w, q


# the path's modes over paged caches: flat, two-stage (blocks of 4, 3 kept), pooled blocks
PAGED_MODES = ({}, {"two_stage": True, "block_size": 4, "n_keep": 3},
               {"two_stage": True, "block_size": 4, "n_keep": 3, "pooled": True})


def check_paged_identity(impl, seed=10):
    """An identity page table is the contiguous cache itself (every mode of the path)."""
    rng = np.random.default_rng(seed)
    L, k_idx, kc, vc, _, _, _, _, q_idx, w, q = _paged_case(rng, 6, 8, 0)
    r = []
    for modes in PAGED_MODES:
        for p, k in ((L - 1, 12), (20, 30), (0, 4)):
            if modes.get("pooled"):
                k = modes["n_keep"] * modes["block_size"]
            a = impl.forward_row(q_idx, k_idx, w, p, k, q_row=q, k_cache=kc, v_cache=vc, **modes)
            b = impl.forward_row_paged(q_idx, k_idx, w, p, k, np.arange(6), 8, q_row=q, k_pool=kc, v_pool=vc,
                                       **modes)
            r.append(_ok(np.array_equal(a["J"], b["J"]) and np.array_equal(a["out"], b["out"])
                         and np.array_equal(a["lse"], b["lse"]), f"identity pages p={p} {modes}"))
    return _all(r)


def check_paged_permutation(impl, seed=11):
    """Pages scattered over a larger pool: the same selection on logical keys, J mapped
    through the page table, the same attention result."""
    rng = np.random.default_rng(seed)
    r = []
    for page_size, n_pages, spare in ((4, 9, 5), (16, 5, 3)):
        L, k_idx, kc, vc, perm, pk, pkc, pvc, q_idx, w, q = _paged_case(rng, n_pages, page_size, spare)
        for modes in PAGED_MODES:
            for p, k in ((L - 1, 10), (L // 2, 7), (3, 9)):
                if modes.get("pooled"):
                    k = modes["n_keep"] * modes["block_size"]
                a = impl.forward_row(q_idx, k_idx, w, p, k, q_row=q, k_cache=kc, v_cache=vc, **modes)
                b = impl.forward_row_paged(q_idx, pk, w, p, k, perm, page_size, q_row=q, k_pool=pkc, v_pool=pvc,
                                           **modes)
                Ja = a["J"]
                want = np.where(Ja >= 0, perm[np.maximum(Ja, 0) // page_size] * page_size
                                + np.maximum(Ja, 0) % page_size, -1)
                ok = (np.array_equal(b["J_logical"], Ja) and np.array_equal(b["J"], want)
                      and np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"]))
                if "kept" in a:
                    ok = ok and np.array_equal(a["kept"], b["kept"])
                r.append(_ok(ok, f"scattered pages P={page_size} p={p} {modes}"))
    return _all(r)


# ---------------------------------------------------------------- semantic search (LSA Flat)
# [LSA] §3.1 "Semantic Clustering", §3.2 "Semantic Search".  Pinned by: closed forms of the
# normalisation and pooling, scipy's Ward linkage (the full hierarchy; Ward's criterion is
# reducible, so merging mutual-cheapest pairs in rounds gives the same clusters as the
# sequential algorithm), the rise of the sum of squared distances computed from the members
# in fp64, hand-worked merge and expansion cases, and the reduction to token-level top-k.

def _sem_keys(rng, n, d=64, scale=1.0):
    return impl_bf16(rng.standard_normal((n, d)) * scale)


def impl_bf16(x):
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def check_sem_normalize_pool(impl, seed=20):
    rng = np.random.default_rng(seed)
    r = []
    x = _sem_keys(rng, 64, scale=3.0)
    y = impl.sem_normalize(x)
    n64 = np.sqrt((y.astype(np.float64) ** 2).sum(1))
    r.append(_ok(np.abs(n64 - 1).max() < 1e-6, f"unit norm {np.abs(n64 - 1).max()}"))
    cos = (y.astype(np.float64) * x).sum(1) / np.sqrt((x.astype(np.float64) ** 2).sum(1))
    r.append(_ok(np.abs(cos - 1).max() < 1e-6, "direction kept"))
    r.append(_ok(np.array_equal(impl.sem_normalize(2 * x), y), "scale by 2 changes no bit"))
    z = np.zeros((3, 64), np.float32)
    r.append(_ok(np.array_equal(impl.sem_normalize(z), z), "zero row stays zero"))
    # pool keys: sums of the normalised keys, whatever the raw norms
    raw = _sem_keys(rng, 32) * np.repeat(rng.integers(1, 50, 32)[:, None], 64, 1).astype(np.float32)
    P = impl.sem_pool_keys(raw, 4)
    x64 = raw.astype(np.float64)
    want = (x64 / np.sqrt((x64 ** 2).sum(1, keepdims=True))).reshape(8, 4, 64).sum(1)
    r.append(_ok(P.shape == (8, 64) and np.abs(P - want).max() < 1e-5, "pool = sum of normalised keys"))
    r.append(_ok(np.array_equal(impl.sem_pool_keys(raw, 1), impl.sem_normalize(raw)), "n_pool 1"))
    # bf16 rounding: nearest, ties to even
    v = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.0e-3], np.float32)
    r.append(_ok(np.array_equal(impl.sem_bf16(v), impl_bf16(v)), "bf16 rounding"))
    return _all(r)


def _clusters_from_log(n, log):
    members = {i: frozenset([i]) for i in range(n)}
    out = {}
    for _, a, b, cost in log:
        members[a] = members[a] | members[b]
        out[members[a]] = cost
    return out


def check_sem_ward_scipy(impl, seed=21):
    from scipy.cluster.hierarchy import linkage
    rng = np.random.default_rng(seed)
    r = []
    for n, d in ((24, 64), (40, 16), (33, 8)):
        P = rng.standard_normal((n, d)).astype(np.float32)
        lab, S, cnt, log = impl.sem_ward(P, 1, n)
        got = _clusters_from_log(n, log)
        Z = linkage(P.astype(np.float64), method="ward")
        mem = {i: frozenset([i]) for i in range(n)}
        want = {}
        for i, (u, v, h, _) in enumerate(Z):
            mem[n + i] = mem[int(u)] | mem[int(v)]
            want[mem[n + i]] = h * h / 2
        same = set(got) == set(want)
        r.append(_ok(same, f"Ward hierarchy n={n}"))
        if same:
            rel = max(abs(got[c] - want[c]) / max(want[c], 1e-12) for c in got)
            r.append(_ok(rel < 1e-3, f"merge costs vs heights n={n}: {rel}"))
        r.append(_ok(len(set(lab.tolist())) == 1 and cnt[0] == n, "one bucket at m=1"))
    return _all(r)


def check_sem_ward_hand(impl):
    # 1-D points on axis 0: mutual pairs (0,1) cost 0.5, (2,3) 0.125, (4,5) 2.
    x = np.array([0, 1, 10, 10.5, 30, 32], np.float32)
    P = np.zeros((6, 8), np.float32)
    P[:, 0] = x
    r = []
    for m, cap, want in ((5, 6, [0, 1, 2, 2, 4, 5]), (4, 6, [0, 0, 2, 2, 4, 5]), (3, 6, [0, 0, 2, 2, 4, 4]),
                         (2, 6, [0, 0, 0, 0, 4, 4]), (1, 6, [0] * 6), (2, 2, [0, 0, 2, 2, 4, 4])):
        lab, S, cnt, log = impl.sem_ward(P, m, cap)
        r.append(_ok(lab.tolist() == want, f"m={m} cap={cap}: {lab.tolist()}"))
    lab, S, cnt, log = impl.sem_ward(P, 2, 6)
    costs = [(a, b, c) for _, a, b, c in log]
    r.append(_ok(costs[:3] == [(0, 1, 0.5), (2, 3, 0.125), (4, 5, 2.0)] and costs[3][:2] == (0, 2)
                 and abs(costs[3][2] - 95.0625) < 1e-4, f"costs {costs}"))
    r.append(_ok(S[0, 0] == 21.5 and cnt[0] == 4 and S[4, 0] == 62, "sums and sizes"))
    return _all(r)


def check_sem_ward_invariants(impl, seed=22):
    rng = np.random.default_rng(seed)
    r = []
    P = impl.sem_pool_keys(_sem_keys(rng, 512), 4)
    for m, cap in ((64, 8), (32, 8), (16, 32)):
        lab, S, cnt, log = impl.sem_ward(P, m, cap)
        ids = sorted(set(lab.tolist()))
        sizes = [int((lab == b).sum()) for b in ids]
        r.append(_ok(len(ids) == m and max(sizes) <= cap, f"m={m} cap={cap}: {len(ids)} {max(sizes)}"))
        r.append(_ok(all(b == int(np.nonzero(lab == b)[0][0]) for b in ids), "id = lowest pool key"))
        s64 = {b: P[lab == b].astype(np.float64).sum(0) for b in ids}
        r.append(_ok(all(np.abs(S[b] - s64[b]).max() < 1e-4 for b in ids), "bucket sum = member sum"))
        # each merge's cost = rise of the sum of squared distances of the members (fp64)
        mem = {i: [i] for i in range(P.shape[0])}
        worst = 0.0
        for _, a, b, cost in log:
            A, Bm = P[mem[a]].astype(np.float64), P[mem[b]].astype(np.float64)
            U = np.vstack([A, Bm])
            sse = lambda X: ((X - X.mean(0)) ** 2).sum()
            rise = sse(U) - sse(A) - sse(Bm)
            worst = max(worst, abs(cost - rise) / max(rise, 1e-6))
            mem[a] = mem[a] + mem[b]
        r.append(_ok(worst < 1e-3, f"cost = SSE rise ({worst})"))
    # well separated blobs of `cap` pool keys come back as the buckets
    cen = rng.standard_normal((8, 64)) * 10
    order = rng.permutation(32)
    Pb = (cen[np.arange(32) // 4] + 0.01 * rng.standard_normal((32, 64)))[order].astype(np.float32)
    lab, _, _, _ = impl.sem_ward(Pb, 8, 4)
    blob = (np.arange(32) // 4)[order]
    r.append(_ok(all(len(set(blob[lab == b])) == 1 and (lab == b).sum() == 4 for b in set(lab.tolist())),
                 "blobs recovered"))
    return _all(r)


def _hand_cache():
    # 3 cluster blocks of 8 keys, 2 buckets each (the bucket cache written out by hand)
    table = np.array([[0, 1, 4, 5, 2, 3, 6, 7], [8, 9, 10, 11, 12, 13, 14, 15],
                      [16, 17, 20, 21, 18, 19, 22, 23]])
    offsets = np.array([[0, 4, 8]] * 3)
    a = np.array([0.125, 0.5, 0.875, 0.25, 0.875, 0.75], np.float32)
    cent = np.zeros((3, 2, 4), np.float32)
    cent[:, :, 0] = a.reshape(3, 2)
    return {"centroids": cent, "table": table, "offsets": offsets, "n_cluster": 8}


def check_sem_select_hand(impl):
    c = _hand_cache()
    q = np.array([3, 0, 0, 0], np.float32)
    r = []
    # p = 26: own block 3; window 19..26; b2 and b4 tie (0.875), the lower id first
    got = impl.semantic_select_row(q, c, 26, 7, 4, 2, 8)
    want = [0, 1, 8, 9, 10, 11, 16, 17, 18] + list(range(19, 27))
    r.append(_ok(got["J"].tolist() == want and got["count"] == 17, f"p=26 k=7: {got['J'].tolist()}"))
    r.append(_ok(got["kept"].tolist() == [2, 4, 5, 1], f"kept {got['kept'].tolist()}"))
    got = impl.semantic_select_row(q, c, 26, 7, 2, 2, 8)
    want = [0, 1, 8, 9, 10, 11, 16, 17] + list(range(19, 27)) + [-1]
    r.append(_ok(got["J"].tolist() == want and got["count"] == 16, f"p=26 top-2: {got['J'].tolist()}"))
    got = impl.semantic_select_row(q, c, 10, 7, 4, 2, 8)
    want = [0, 1, 2] + list(range(3, 11)) + [-1] * 6
    r.append(_ok(got["J"].tolist() == want and got["count"] == 11, f"p=10: {got['J'].tolist()}"))
    got = impl.semantic_select_row(q, c, 5, 7, 4, 2, 8)
    r.append(_ok(got["J"].tolist() == list(range(6)) + [-1] * 11 and got["count"] == 6, "p=5: window only"))
    got = impl.semantic_select_row(q, c, -1, 7, 4, 2, 8)
    r.append(_ok(got["count"] == 0 and (got["J"] == -1).all(), "padding row"))
    s = impl.sem_scores(np.array([1, 0, 0, 0], np.float32), c["centroids"].reshape(6, 4))
    r.append(_ok(s.tolist() == [0.125, 0.5, 0.875, 0.25, 0.875, 0.75], "scores"))
    key = impl.sem_order_key(np.array([-2.0, -0.0, 0.0, 1e-30, 3.0], np.float32))
    r.append(_ok(np.all(np.diff(key.astype(np.int64)) > 0), "order key"))
    return _all(r)


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)


def check_sem_cluster_hand(impl):
    """The cache entry of the hand-clustered block: merge rounds, bucket order, each
    bucket's keys ascending, offsets, and the centroids' bf16 bit patterns."""
    g = _load_golden()["semantic_cluster"]
    keys = np.array(g["keys"], np.float32)
    r = []
    P = impl.sem_pool_keys(keys, g["n_pool"])
    _, _, _, log = impl.sem_ward(P, g["m"], g["n_max"] // g["n_pool"])
    r.append(_ok([[a, b, c] for a, b, c, _ in log] == g["merge_log"], f"merge rounds {log}"))
    cent, table, off = impl.sem_cluster_block(keys, g["n_pool"], g["m"], g["n_max"])
    r.append(_ok(np.asarray(table).tolist() == g["table"], f"table {np.asarray(table).tolist()}"))
    r.append(_ok(np.asarray(off).tolist() == g["offsets"], f"offsets {np.asarray(off).tolist()}"))
    want = [[int(h, 16) for h in row] for row in g["centroid_bf16_bits"]]
    cent = np.asarray(cent, np.float32)
    exact = cent.shape == (4, 4) and (cent.view(np.uint32) & 0xFFFF).max() == 0
    r.append(_ok(exact and _bf16_bits(cent).tolist() == want, f"centroid bits {cent.tolist()}"))
    # the same entry through the whole-sequence cache, its first key offset applied
    c = impl.bucket_cache(np.vstack([keys, keys]), g["n_cluster"], g["n_pool"], g["n_bavg"], g["n_max"])
    r.append(_ok(np.asarray(c["table"][1]).tolist() == [j + 16 for j in g["table"]], "second block's table"))
    return _all(r)


def check_sem_expand_cut_hand(impl):
    """Expansion whose cut falls inside a multi-key bucket, over the hand-made cache."""
    g = _load_golden()["semantic_cluster"]
    e = g["expansion"]
    keys = np.vstack([np.array(g["keys"], np.float32), np.eye(4, dtype=np.float32)[[0, 1, 2, 3, 0, 1, 2, 3]]])
    c = impl.bucket_cache(keys, g["n_cluster"], g["n_pool"], g["n_bavg"], g["n_max"])
    r = []
    for cs in e["cases"]:
        got = impl.semantic_select_row(np.array(e["q"], np.float32), c, e["p"], cs["k"], cs["p_top"],
                                       cs["n_sink"], cs["n_w"])
        want = cs["J"] + [-1] * (cs["n_sink"] + cs["k"] + cs["n_w"] - len(cs["J"]))
        r.append(_ok(got["J"].tolist() == want and got["count"] == cs["count"],
                     f"k={cs['k']} n_w={cs['n_w']}: {got['J'].tolist()}"))
    return _all(r)


def check_sem_token_reduction(impl, seed=23):
    """One key per bucket (n_pool = 1, m = n_cluster, no merge) and p = k: the long-range
    keys are the exact top-k of the cosine scores over the keys of the earlier cluster
    blocks, less those in the sink or the window."""
    rng = np.random.default_rng(seed)
    r = []
    n_c, d = 32, 64
    keys = _sem_keys(rng, 8 * n_c)
    c = impl.bucket_cache(keys, n_c, 1, 1, 2)
    k64 = keys.astype(np.float64)
    kn = impl_bf16(k64 / np.sqrt((k64 ** 2).sum(1, keepdims=True)))
    for p, k, n_sink, n_w in ((8 * n_c - 1, 20, 4, n_c), (5 * n_c + 3, 37, 0, n_c), (3 * n_c, 50, 2, 2 * n_c)):
        q = _sem_keys(rng, 1)[0]
        q64 = q.astype(np.float64)
        qn = impl_bf16(q64 / np.sqrt((q64 ** 2).sum())).astype(np.float64)
        nb = p // n_c
        w0 = max(0, p - n_w + 1)
        # the k best keys of the earlier blocks are the k selected buckets; the expansion
        # then drops those in the sink or the window
        sc = kn[: nb * n_c].astype(np.float64) @ qn
        top = {j for j in np.argsort(-sc, kind="stable")[:k].tolist() if n_sink <= j < w0}
        got = impl.semantic_select_row(q, c, p, k, k, n_sink, n_w)
        J = got["J"][got["J"] >= 0]
        lr = set(J.tolist()) - set(range(min(n_sink, p + 1))) - set(range(w0, p + 1))
        r.append(_ok(lr == top, f"p={p} k={k}: {len(lr ^ top)} differ"))
    return _all(r)


def check_sem_invariants(impl, seed=24):
    rng = np.random.default_rng(seed)
    r = []
    n_c = 512
    keys = _sem_keys(rng, 6 * n_c)
    c = impl.bucket_cache(keys, n_c, 4, 8, 32)
    m = 64
    r.append(_ok(all(sorted(c["table"][b].tolist()) == list(range(b * n_c, (b + 1) * n_c)) for b in range(6)),
                 "table holds every key of its block once"))
    sz = np.diff(c["offsets"], axis=1)
    r.append(_ok(sz.min() >= 4 and sz.max() <= 32 and (sz % 4 == 0).all(), "bucket sizes"))
    n64 = np.sqrt((c["centroids"].astype(np.float64) ** 2).sum(-1))
    r.append(_ok(np.abs(n64 - 1).max() < 1e-2, "unit centroids"))
    for p, k, pt in ((6 * n_c - 1, 300, 64), (6 * n_c - 1, 300, 16), (2 * n_c + 7, 200, 64), (n_c, 50, 8)):
        q = _sem_keys(rng, 1)[0]
        g = impl.semantic_select_row(q, c, p, k, pt, 4, n_c)
        J = g["J"][: g["count"]]
        w0 = max(0, p - n_c + 1)
        ok = (np.all(np.diff(J) > 0) and (g["J"][g["count"]:] == -1).all() and J[-1] == p
              and set(range(4)) <= set(J.tolist()) and set(range(w0, p + 1)) <= set(J.tolist()))
        r.append(_ok(ok, f"J shape p={p}"))
        lr = [j for j in J.tolist() if 4 <= j < w0]
        kept = g["kept"]
        bk = {}
        for i, b in enumerate(kept):
            blk, loc = divmod(int(b), m)
            for j in c["table"][blk, c["offsets"][blk, loc]:c["offsets"][blk, loc + 1]]:
                bk[int(j)] = i
        avail = sum(1 for j in bk if 4 <= j < w0)
        r.append(_ok(all(j in bk for j in lr) and len(lr) == min(k, avail), f"long-range keys p={p}"))
        if lr:
            # best first: every bucket ranked before the last one used is taken whole
            last = max(bk[j] for j in lr)
            whole = all(j in lr for j, i in bk.items() if i < last and 4 <= j < w0)
            r.append(_ok(whole, f"buckets taken best first p={p}"))
        s = g["scores"]
        kk = impl.sem_order_key(s).astype(np.int64)
        rest = np.setdiff1d(np.arange(s.shape[0]), kept)
        r.append(_ok(len(kept) == min(pt, s.shape[0]) and (rest.size == 0 or kk[kept].min() >= kk[rest].max()),
                     "top-p buckets"))
    return _all(r)


ALL_CHECKS = [
    check_scores_hand, check_scores_closed_forms, check_scores_invariances, check_scores_bound,
    check_topk_hand, check_topk_bruteforce, check_topk_special,
    check_blocks_hand, check_block_reps_sum, check_block_keep_bruteforce,
    check_two_stage_reductions, check_two_stage_invariants,
    check_attention_hand, check_attention_dense, check_attention_special,
    check_paged_hand, check_paged_identity, check_paged_permutation,
    check_pooled_hand, check_pooled_dense,
    check_sem_normalize_pool, check_sem_ward_scipy, check_sem_ward_hand, check_sem_ward_invariants,
    check_sem_select_hand, check_sem_token_reduction, check_sem_invariants,
    check_sem_cluster_hand, check_sem_expand_cut_hand,
]
