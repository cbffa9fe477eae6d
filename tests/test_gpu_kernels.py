"""GPU parity of every C-ABI call against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails, plus the
edge cases of the method (empty / short rows, ties, padding, degenerate lists)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import AttnErr, dev, np64, topk_certificate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lsa():
    import learned_top_sparse_amd as m
    m.lib()  # raises if liblsa.so is missing: no fallback
    return m


def _inputs(wl, seed=0, pos=None):
    inp = synthetic.make_inputs(wl.replace(seed=seed), "cpu")
    if pos is not None:
        inp["q_pos"] = torch.as_tensor(pos, dtype=torch.int32).reshape(wl.B, wl.n_q).contiguous()
    return inp, {k: v.to(dev()) for k, v in inp.items()}


def _flat_oracle_rows(inp, k, with_attn=True, rows=None):
    qi, ki, w, qp = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["w"].numpy(), inp["q_pos"].numpy()
    B, n_q = qp.shape
    q = np64(inp["q"]) if with_attn else None
    kk = np64(inp["k"]) if with_attn else None
    vv = np64(inp["v"]) if with_attn else None
    scale = 1.0 / math.sqrt(inp["q"].shape[-1]) if with_attn else None
    out = {}
    for b, i in (rows or [(b, i) for b in range(B) for i in range(n_q)]):
        wr = w[b, i] if w.ndim == 3 else w
        out[(b, i)] = oracle.forward_row(qi[b, i], ki[b], wr, int(qp[b, i]), k,
                                         q_row=None if q is None else q[b, i],
                                         k_cache=None if kk is None else kk[b],
                                         v_cache=None if vv is None else vv[b], scale=scale)
    return out


# ----------------------------------------------------------------------------- indexer
@pytest.mark.parametrize("case", [
    # (H_I, d_I, B, n_q, L, positions, w_per_query)
    (4, 64, 1, 1024, 1024, "causal", False),      # the tiny prefill workload
    (64, 128, 1, 37, 1000, "random", False),      # ragged key tail, ragged query tile
    (20, 64, 2, 50, 777, "tail", False),          # heads not a multiple of 16
    (64, 128, 3, 1, 5000, "last", False),         # decode-shaped (one query per sequence)
    (48, 128, 1, 16, 300, "random", True),        # per-query head weights
    (1, 128, 1, 9, 130, "random", False),         # a single indexer head
    (64, 128, 1, 8, 70000, "last", False),        # long rows, several spans
])
def test_index_scores_exact(lsa, case):
    H_I, d_I, B, n_q, L, mode, wpq = case
    wl = synthetic.Workload("t", B=B, n_q=n_q, L=L, q_pos0=0, H_I=H_I, d_I=d_I, k=16, H_q=8)
    rng = np.random.default_rng(H_I * 1000 + L)
    if mode == "causal":
        pos = np.arange(n_q)[None].repeat(B, 0)
    elif mode == "random":
        pos = rng.integers(0, L, size=(B, n_q))
    elif mode == "tail":
        pos = (L - n_q + np.arange(n_q))[None].repeat(B, 0)
    else:
        pos = np.full((B, n_q), L - 1)
    inp, g = _inputs(wl, seed=3, pos=pos)
    if wpq:
        inp["w"] = torch.randint(1, 17, (B, n_q, H_I), generator=torch.Generator().manual_seed(5), dtype=torch.int32)
        g["w"] = inp["w"].to(dev())
    S = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"])
    S = S.cpu().numpy()
    qi, ki, w = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["w"].numpy()
    for b in range(B):
        for i in range(n_q):
            p = int(pos[b, i])
            want = oracle.index_scores(qi[b, i], ki[b], w[b, i] if wpq else w, p)
            assert np.array_equal(S[b, i, : p + 1], want), f"row {(b, i)} p={p}"


def test_index_scores_extreme_values(lsa):
    """Largest magnitudes of the workload ranges: q, k = +-64, w = 16 (scores up to 2^29)."""
    B, n_q, L, H, d = 1, 8, 200, 64, 128
    rng = np.random.default_rng(11)
    q = rng.choice([-64, 64], size=(B, n_q, H, d)).astype(np.int8)
    k = rng.choice([-64, 64], size=(B, L, d)).astype(np.int8)
    k[0, :10] = 64
    q[0, 0] = 64
    w = np.full(H, 16, np.int32)
    pos = np.full((B, n_q), L - 1, np.int32)
    t = lambda a: torch.from_numpy(a).to(dev())
    S = lsa.lsa_index_scores(t(q), t(k), t(w), t(pos)).cpu().numpy()
    for i in range(n_q):
        assert np.array_equal(S[0, i], oracle.index_scores(q[0, i], k[0], w, L - 1))
    assert S[0, 0, 0] == H * 16 * d * 64 * 64


# ----------------------------------------------------------------------------- top-k
def _topk_case(kind, n_rows, L, rng):
    if kind == "random":
        return rng.integers(-2 ** 31, 2 ** 31, size=(n_rows, L), dtype=np.int64).astype(np.int32)
    if kind == "ties3":
        return rng.integers(-1, 2, size=(n_rows, L)).astype(np.int32)
    if kind == "equal":
        return np.zeros((n_rows, L), np.int32)
    if kind == "increasing":
        return np.tile(np.arange(L, dtype=np.int32), (n_rows, 1))
    if kind == "decreasing":
        return np.tile(-np.arange(L, dtype=np.int32), (n_rows, 1))
    if kind == "extremes":
        return rng.choice(np.array([-2 ** 31, -1, 0, 2 ** 31 - 1], dtype=np.int64), size=(n_rows, L)).astype(np.int32)
    if kind == "indexer_like":
        return np.clip(rng.normal(3.4e6, 7e5, size=(n_rows, L)), 0, 2 ** 29).astype(np.int32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["random", "ties3", "equal", "increasing", "decreasing", "extremes",
                                  "indexer_like"])
@pytest.mark.parametrize("k", [1, 7, 64, 2048])
def test_topk_exact(lsa, kind, k):
    rng = np.random.default_rng(hash((kind, k)) % 2 ** 32)
    L, n_rows = 5000, 24
    S = _topk_case(kind, n_rows, L, rng)
    pos = rng.integers(0, L, size=n_rows).astype(np.int32)
    pos[:4] = [0, k - 1, k, L - 1]
    pos = np.clip(pos, 0, L - 1)
    Sg = torch.from_numpy(S).reshape(1, n_rows, L).to(dev())
    pg = torch.from_numpy(pos).reshape(1, n_rows).to(dev())
    J, cnt = lsa.lsa_topk(Sg, pg, k, L)
    J, cnt = J.cpu().numpy()[0], cnt.cpu().numpy()[0]
    for r in range(n_rows):
        p = int(pos[r])
        want, wc = oracle.topk(S[r, : p + 1], np.arange(p + 1), k)
        assert np.array_equal(J[r], want), f"{kind} k={k} row {r} p={p}"
        assert cnt[r] == wc


@pytest.mark.parametrize("kind,L,k", [("equal", 262144, 2048), ("ties3", 131073, 2048),
                                      ("indexer_like", 262144, 2048), ("increasing", 200000, 4096),
                                      ("random", 40000, 4096)])
def test_topk_long_rows(lsa, kind, L, k):
    """Long rows: both the LDS-list path and the global fallback (heavy ties) are exact."""
    rng = np.random.default_rng(L + k)
    n_rows = 6
    S = _topk_case(kind, n_rows, L, rng)
    pos = np.array([L - 1, L - 2, L // 2, k, k - 1, 3 * L // 4], np.int32)
    Sg = torch.from_numpy(S).reshape(1, n_rows, L).to(dev())
    J, _ = lsa.lsa_topk(Sg, torch.from_numpy(pos).reshape(1, n_rows).to(dev()), k, L)
    J = J.cpu().numpy()[0]
    for r in range(n_rows):
        p = int(pos[r])
        want, _ = oracle.topk(S[r, : p + 1], np.arange(p + 1), k)
        assert np.array_equal(J[r], want), f"{kind} row {r}"


@pytest.mark.parametrize("kind", ["indexer_like", "equal", "ties3", "random"])
def test_topk_split_rows_match_single_workgroup(lsa, kind):
    """Decode-shaped rows: the several-workgroups-per-row path equals the one-workgroup path and the oracle."""
    rng = np.random.default_rng(13)
    L, k, n_rows = 131073, 2048, 9
    S = _topk_case(kind, n_rows, L, rng)
    pos = np.array([L - 1, L - 2, 100000, 40000, 32767, 8191, 2047, 2048, 0], np.int32)
    Sg = torch.from_numpy(S).reshape(1, n_rows, L).to(dev())
    pg = torch.from_numpy(pos).reshape(1, n_rows).to(dev())
    J1, c1 = lsa.lsa_topk(Sg, pg, k, L, use_ws=True)
    J2, c2 = lsa.lsa_topk(Sg, pg, k, L, use_ws=False)
    assert torch.equal(J1, J2) and torch.equal(c1, c2)
    J1 = J1.cpu().numpy()[0]
    for r in range(n_rows):
        p = int(pos[r])
        want, _ = oracle.topk(S[r, : p + 1], np.arange(p + 1), k)
        assert np.array_equal(J1[r], want), f"{kind} row {r}"


def test_topk_many_rows_workgroup_variants(lsa):
    """Same rows through the 256-thread and the 1024-thread variants give identical lists."""
    rng = np.random.default_rng(7)
    L, k = 20000, 2048
    S = _topk_case("indexer_like", 8, L, rng)
    pos = np.full(8, L - 1, np.int32)
    Sg = torch.from_numpy(S).reshape(1, 8, L).to(dev())
    J1, _ = lsa.lsa_topk(Sg, torch.from_numpy(pos).reshape(1, 8).to(dev()), k, L)   # 1024 threads
    big = torch.from_numpy(np.repeat(S, 200, axis=0)).reshape(1, 1600, L).to(dev())
    J2, _ = lsa.lsa_topk(big, torch.from_numpy(np.repeat(pos, 200)).reshape(1, 1600).to(dev()), k, L)  # 256
    J1, J2 = J1.cpu().numpy()[0], J2.cpu().numpy()[0]
    for r in range(8):
        want, _ = oracle.topk(S[r], np.arange(L), k)
        assert np.array_equal(J1[r], want)
        assert np.array_equal(J2[200 * r], want)


@pytest.mark.parametrize("bs,n_keep", [(16, 4), (128, 64), (7, 5)])
def test_topk_kept_slots(lsa, bs, n_keep):
    rng = np.random.default_rng(bs * 100 + n_keep)
    n_rows, L, k = 20, 64 * bs, 3 * bs
    n_blk = L // bs
    pos = rng.integers(0, L, size=n_rows).astype(np.int32)
    kept = np.full((n_rows, n_keep), -1, np.int32)
    for r in range(n_rows):
        own = pos[r] // bs
        cnt = rng.integers(1, n_keep + 1)
        cand = rng.choice(max(own, 1), size=min(cnt - 1, own), replace=False) if own > 0 else []
        blocks = np.sort(np.concatenate([np.asarray(cand, np.int64), [own]]))
        kept[r, : len(blocks)] = blocks
    width = n_keep * bs
    S = rng.integers(-5, 6, size=(n_rows, width)).astype(np.int32)
    Sg = torch.from_numpy(S).reshape(1, n_rows, width).to(dev())
    J, cnt = lsa.lsa_topk(Sg, torch.from_numpy(pos).reshape(1, n_rows).to(dev()), k, L,
                          kept_blocks=torch.from_numpy(kept).reshape(1, n_rows, n_keep).to(dev()), block_size=bs)
    J, cnt = J.cpu().numpy()[0], cnt.cpu().numpy()[0]
    for r in range(n_rows):
        slots = np.arange(width)
        blk = kept[r, slots // bs]
        key = blk.astype(np.int64) * bs + slots % bs
        ok = (blk >= 0) & (key <= pos[r])
        want, wc = oracle.topk(S[r, ok], key[ok], k)
        assert np.array_equal(J[r], want), f"row {r}"
        assert cnt[r] == wc
    assert n_blk > 0


# ----------------------------------------------------------------------------- two-stage blocks
@pytest.mark.parametrize("case", [
    # (T, bs, n_keep, H_I, d_I, value range)
    (2048, 16, 4, 4, 64, 64),
    (4096, 128, 8, 64, 128, 64),
    (2048, 16, 6, 8, 128, 1),       # k_idx / q_idx in {-1, 0, 1}: many tied block scores
    (1536, 100, 5, 20, 64, 127),    # block size not a power of two, full int8 range
])
def test_block_reps_and_prefilter(lsa, case):
    T, bs, n_keep, H, d, vr = case
    rng = np.random.default_rng(T + bs)
    n_q = 40
    q = rng.integers(-vr, vr + 1, size=(1, n_q, H, d)).astype(np.int8)
    k = rng.integers(-vr, vr + 1, size=(1, T, d)).astype(np.int8)
    w = rng.integers(1, 17, size=H).astype(np.int32)
    pos = np.sort(rng.integers(0, T, size=n_q)).astype(np.int32)
    pos[:3] = [0, bs - 1, bs]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    n_blocks = T // bs
    reps = lsa.lsa_block_reps(t(k), bs, n_blocks)
    R = oracle.block_reps(k[0], bs)
    assert np.array_equal(reps.cpu().numpy()[0], R)
    kept, bsc = lsa.lsa_block_prefilter(t(q), reps, t(w), t(pos.reshape(1, n_q)), bs, n_keep, return_scores=True)
    kept, bsc = kept.cpu().numpy()[0], bsc.cpu().numpy()[0]
    for i in range(n_q):
        want, want_bs = oracle.block_keep(q[0, i], R, w, int(pos[i]), bs, n_keep)
        own = int(pos[i]) // bs
        assert np.array_equal(bsc[i, :own], want_bs), f"block scores row {i}"
        padded = np.full(n_keep, -1)
        padded[: want.size] = want
        assert np.array_equal(kept[i], padded), f"kept row {i}"


@pytest.mark.parametrize("T", [24576, 49152, 98304])
@pytest.mark.parametrize("mode", ["random", "signed", "ties", "zeros", "bigw", "extreme"])
def test_block_prefilter_long_rows(lsa, mode, T):
    """Prefill-shaped rows over more than 4096 blocks: 6144 blocks take the keep that
    holds the row in registers (read once), 12288 and 24576 the keep that reads each
    row's scores twice (a coarse histogram, then the cut's bin gathered into LDS; its
    256- and 1024-thread forms).  Kept blocks equal the
    oracle's for rows whose cut bin holds a few members (random), scores of both signs
    (signed weights), heavily tied scores (q, k in {-1, 0, 1}), and every score equal
    (rows whose tie outgrows the LDS member list then take the multi-pass fallback,
    shorter ones settle all their ties in LDS).  Block scores equal the oracle's at
    the extremes of their int64 sums too: q = k = -128 with w = 16 over 64 heads (every
    block 2^33) and weights near 2^20."""
    bs, n_keep, d = 4, 256, 128
    H = 64 if mode == "extreme" else 8
    rng = np.random.default_rng({"random": 1, "signed": 2, "ties": 3, "zeros": 4, "bigw": 5, "extreme": 6}[mode] + T)
    n_q = 24
    vr = 1 if mode == "ties" else 64
    q = rng.integers(-vr, vr + 1, size=(1, n_q, H, d)).astype(np.int8)
    if mode == "zeros":
        q[:] = 0
    k = rng.integers(-vr, vr + 1, size=(1, T, d)).astype(np.int8)
    if mode == "extreme":
        q[:] = -128
        k[:] = -128
    if mode == "signed":
        w = rng.integers(-16, 17, size=H)
    elif mode == "bigw":
        w = rng.integers(2 ** 20, 2 ** 21, size=H)
    elif mode == "extreme":
        w = np.full(H, 16)
    else:
        w = rng.integers(1, 17, size=H)
    w = w.astype(np.int32)
    pos = np.sort(rng.integers(4 * 4096, T, size=n_q)).astype(np.int32)
    pos[:4] = [0, 4 * n_keep - 1, 4 * n_keep + 5, 4 * 3000 + 1]  # all kept, one to cut, a short row
    pos[-1] = T - 1
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    reps = lsa.lsa_block_reps(t(k), bs, T // bs)
    R = oracle.block_reps(k[0], bs)
    kept, bsc = lsa.lsa_block_prefilter(t(q), reps, t(w), t(pos.reshape(1, n_q)), bs, n_keep, return_scores=True)
    kept, bsc = kept.cpu().numpy()[0], bsc.cpu().numpy()[0]
    for i in range(n_q):
        want, want_bs = oracle.block_keep(q[0, i], R, w, int(pos[i]), bs, n_keep)
        own = int(pos[i]) // bs
        assert np.array_equal(bsc[i, :own], want_bs), f"block scores row {i}"
        padded = np.full(n_keep, -1)
        padded[: want.size] = want
        assert np.array_equal(kept[i], padded), f"kept row {i} (p = {pos[i]})"
    if mode == "signed":
        assert (bsc < 0).any() and (bsc > 0).any()
    if mode == "extreme":
        assert bsc[-1, 0] == H * 16 * d * 128 * 512


# ----------------------------------------------------------------------------- attention
def _attn_inputs(B, n_q, L, H, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, n_q, H, 128), generator=g).to(torch.bfloat16)
    k = torch.randn((B, L, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, L, 128), generator=g).to(torch.bfloat16)
    return q, k, v


def _attn_oracle(q, k, v, J, scale):
    qn, kn, vn, Jn = np64(q), np64(k), np64(v), J.cpu().numpy()
    B, n_q, H, _ = qn.shape
    out = np.zeros((B, n_q, H, 128))
    lse = np.zeros((B, n_q, H))
    for b in range(B):
        for i in range(n_q):
            out[b, i], lse[b, i] = oracle.sparse_attention(qn[b, i], kn[b], vn[b], Jn[b, i], scale)
    return out, lse


@pytest.mark.parametrize("H", [16, 8, 5])
@pytest.mark.parametrize("n_split", [1, 3, 0])
def test_sparse_attn_random_lists(lsa, H, n_split):
    B, n_q, L, k = 2, 24, 3000, 300
    q, k_, v = _attn_inputs(B, n_q, L, H, seed=H + n_split)
    rng = np.random.default_rng(H)
    J = np.full((B, n_q, k), -1, np.int32)
    for b in range(B):
        for i in range(n_q):
            n = rng.integers(0, k + 1) if i % 3 else k
            sel = np.sort(rng.choice(L, size=n, replace=False))
            J[b, i, :n] = sel
            if i % 5 == 1 and n > 4:   # -1 entries in the middle and out-of-range ids are skipped
                J[b, i, 2] = -1
                J[b, i, 3] = L + 7
    Jt = torch.from_numpy(J)
    scale = 1 / math.sqrt(128)
    out, lse = lsa.lsa_sparse_attn(q.to(dev()), k_.to(dev()), v.to(dev()), Jt.to(dev()), scale, n_split=n_split)
    J2 = J.copy()
    J2[(J2 >= L)] = -1
    want, want_lse = _attn_oracle(q, k_, v, torch.from_numpy(J2), scale)
    err = AttnErr()
    err.add(np64(out), want)
    err.check()
    lse = lse.cpu().numpy()
    fin = np.isfinite(want_lse)
    assert np.all(np.isneginf(lse[~fin]))
    assert np.max(np.abs(lse[fin] - want_lse[fin])) < 1e-3
    empty = (J2 < 0).all(-1)
    assert np.all(np64(out)[empty] == 0)


@pytest.mark.parametrize("n_split", [1, 2, 3, 5, 12, 0])
def test_sparse_attn_split_forms(lsa, n_split):
    """Every launch form on one list length (35 tiles, the last one ragged): one unit per
    row with pipelined waves (1), split units of more than 16 tiles, pipelined (2), and
    the one-tile form with 16, 8 and 4 waves (3, 5, 12 splits), plus the automatic count."""
    B, n_q, L, H, k = 3, 2, 5000, 16, 1100
    q, k_, v = _attn_inputs(B, n_q, L, H, seed=40 + n_split)
    rng = np.random.default_rng(n_split)
    J = np.full((B, n_q, k), -1, np.int32)
    for b in range(B):
        for i in range(n_q):
            n = k if (b + i) % 2 == 0 else int(rng.integers(1, k))
            J[b, i, :n] = rng.choice(L, size=n, replace=False)
    Jt = torch.from_numpy(J)
    scale = 1 / math.sqrt(128)
    out, lse = lsa.lsa_sparse_attn(q.to(dev()), k_.to(dev()), v.to(dev()), Jt.to(dev()), scale, n_split=n_split)
    want, want_lse = _attn_oracle(q, k_, v, Jt, scale)
    err = AttnErr()
    err.add(np64(out), want)
    err.check()
    assert np.max(np.abs(lse.cpu().numpy() - want_lse)) < 1e-3


def test_sparse_attn_degenerate_lists(lsa):
    B, n_q, L, H = 1, 6, 500, 16
    q, k, v = _attn_inputs(B, n_q, L, H, seed=1)
    q[0, 3] = q[0, 2]                    # same query for the plain and the reversed list
    J = np.full((B, n_q, 64), -1, np.int32)
    J[0, 0, 0] = 17                      # one key: softmax weight 1, output = V[17] exactly
    J[0, 1, 40] = 499                    # one key late in the list
    J[0, 2, :] = np.arange(64)           # plain list
    J[0, 3, :] = np.arange(64)[::-1]     # same keys, reversed order
    J[0, 4, :] = 5                       # one key listed 64 times
    out, _ = lsa.lsa_sparse_attn(q.to(dev()), k.to(dev()), v.to(dev()), torch.from_numpy(J).to(dev()))
    out = out.cpu()
    assert torch.equal(out[0, 0], v[0, 17].unsqueeze(0).expand(H, 128))
    assert torch.equal(out[0, 1], v[0, 499].unsqueeze(0).expand(H, 128))
    assert torch.equal(out[0, 4], v[0, 5].unsqueeze(0).expand(H, 128))
    d = (out[0, 2].float() - out[0, 3].float()).abs().max().item()
    assert d <= 2 ** -7, f"order dependence {d}"
    assert torch.all(out[0, 5] == 0)


def test_sparse_attn_dense_equivalence(lsa):
    """k >= t+1: the list holds every causal key, so the result is dense causal attention."""
    T, H = 200, 16
    q, k, v = _attn_inputs(1, T, T, H, seed=2)
    J = np.full((1, T, 256), -1, np.int32)
    for t in range(T):
        J[0, t, : t + 1] = np.arange(t + 1)
    out, _ = lsa.lsa_sparse_attn(q.to(dev()), k.to(dev()), v.to(dev()), torch.from_numpy(J).to(dev()))
    import torch.nn.functional as F
    qd = q.double()[0].permute(1, 0, 2).unsqueeze(0)
    kd = k.double()[0][None, None].expand(1, H, T, 128)
    vd = v.double()[0][None, None].expand(1, H, T, 128)
    dense = F.scaled_dot_product_attention(qd, kd, vd, is_causal=True, scale=1 / math.sqrt(128))
    dense = dense[0].permute(1, 0, 2).numpy()
    err = AttnErr()
    err.add(np64(out)[0], dense)
    err.check()


# ----------------------------------------------------------------------------- whole path
def test_forward_tiny_prefill_all_rows(lsa):
    wl = synthetic.WORKLOADS["tiny_prefill_1k"]
    inp, g = _inputs(wl)
    res = lsa.lsa_forward(g, k_top=wl.k)
    want = _flat_oracle_rows(inp, wl.k)
    J, cnt, out = res["idx"].cpu().numpy(), res["count"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for (b, i), r in want.items():
        assert np.array_equal(J[b, i], r["J"]), f"row {i}"
        assert cnt[b, i] == r["count"]
        err.add(out[b, i], r["out"], (b, i))
    err.check()


@pytest.mark.parametrize("chunk_rows", [0, 100, 333])
def test_forward_chunking_identical(lsa, chunk_rows):
    """Score chunks of any size give bit-identical lists and outputs."""
    wl = synthetic.WORKLOADS["tiny_prefill_1k"].replace(H_I=64, d_I=128, k=96, H_q=16)
    _, g = _inputs(wl, seed=4)
    # the automatic attention split depends on the chunk's row count; pin it for bit identity
    ref = lsa.lsa_forward(g, k_top=wl.k, chunk_rows=0, attn_split=1)
    res = lsa.lsa_forward(g, k_top=wl.k, chunk_rows=chunk_rows, attn_split=1)
    assert torch.equal(ref["idx"], res["idx"])
    assert torch.equal(ref["out"], res["out"])


@pytest.mark.parametrize("kind", ["random", "zero_queries", "concentrated"])
def test_forward_thresholded_selection_modes(lsa, kind):
    """Flat prefill rows longer than 8k keys take the thresholded selection (a threshold
    from sampled scores, candidate lists, the exact top-k from the lists, the score table
    for lists that fall short or overflow).  Every mode gives the score table's lists,
    counts and outputs bit for bit, and the oracle's on sampled rows: auto; every
    thresholded row forced to fall short; forced to overflow.  Rows up to 4096 keys
    (the score table) mix in, the 4097-key row is the shortest list row; half the queries all-zero (every score 0: the lists
    overflow); or every query's best keys in one 600-key window."""
    k = 512
    wl = synthetic.Workload("thr", B=2, n_q=96, L=24000, q_pos0=0, H_I=64, d_I=128, k=k, H_q=16)
    pos = np.linspace(0, 23999, 96).astype(np.int64)
    pos[:8] = [0, 300, 511, 512, 2047, 2048, 4095, 4096]
    inp, _ = _inputs(wl, seed=21, pos=np.tile(pos, 2))
    if kind == "zero_queries":
        inp["q_idx"][:, ::2] = 0
    elif kind == "concentrated":
        gen = torch.Generator().manual_seed(8)
        vdir = torch.randint(-64, 65, (128,), generator=gen, dtype=torch.int64)
        inp["q_idx"][:, :, 0, :] = vdir.to(torch.int8)
        noise = torch.randint(-3, 4, (600, 128), generator=gen, dtype=torch.int64)
        inp["k_idx"][:, 5000:5600] = (vdir + noise).clamp(-128, 127).to(torch.int8)
    g = {kk: v.to(dev()) for kk, v in inp.items()}
    ws = lsa.lsa_forward_workspace_size(g, k)
    assert lsa.lsa_forward_stages(g, k, ws)[0] == "sample"
    ref = lsa.lsa_forward(g, k_top=k, select="table", attn_split=1)
    for mode in ("auto", "force_short", "force_overflow"):
        res = lsa.lsa_forward(g, k_top=k, select=mode, attn_split=1)
        assert torch.equal(res["idx"], ref["idx"]), f"{kind} {mode}"
        assert torch.equal(res["count"], ref["count"]), f"{kind} {mode}"
        assert torch.equal(res["out"], ref["out"]), f"{kind} {mode}"
    rows = [(0, 0), (0, 3), (0, 6), (0, 7), (1, 50), (1, 95)]
    want = _flat_oracle_rows(inp, k, with_attn=False, rows=rows)
    J = ref["idx"].cpu().numpy()
    for (b, i), r in want.items():
        assert np.array_equal(J[b, i], r["J"]), f"{kind} row {(b, i)}"


def test_forward_decode_small(lsa):
    wl = synthetic.Workload("dec", B=5, n_q=1, L=9000, q_pos0=8999, H_I=64, d_I=128, k=512, H_q=16)
    inp, g = _inputs(wl, seed=5)
    res = lsa.lsa_forward(g, k_top=wl.k)
    want = _flat_oracle_rows(inp, wl.k)
    J, out = res["idx"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for (b, i), r in want.items():
        assert np.array_equal(J[b, i], r["J"]), f"seq {b}"
        err.add(out[b, i], r["out"], (b, i))
    err.check()


@pytest.mark.parametrize("H_I", [64, 20])
def test_forward_decode_fused_selection(lsa, H_I):
    """Decode rows: lsa_forward lets the indexer leave each span's histogram and
    candidate list (stages index_select, topk, sparse_attn).  Its lists equal the
    separate calls' (score table, then lsa_topk) bit for bit, and the oracle's on
    sampled rows; rows of at most k candidates mix in."""
    L, k = 40000, 1024
    pos = [39999, 30000, 1023, 500, 33333, 39998]
    wl = synthetic.Workload("decfused", B=len(pos), n_q=1, L=L, q_pos0=0, H_I=H_I, d_I=128, k=k, H_q=16)
    inp, g = _inputs(wl, seed=11, pos=pos)
    ws_bytes = lsa.lsa_forward_workspace_size(g, k)
    assert lsa.lsa_forward_stages(g, k, ws_bytes) == ["index_select", "topk", "sparse_attn"]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    res = lsa.lsa_forward(g, k_top=k, stage_events=evs)
    torch.cuda.synchronize()
    assert all(evs[i].elapsed_time(evs[i + 1]) >= 0 for i in range(3))
    ld = ((L + 63) // 64) * 64
    sc = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"], ld=ld)
    for use_ws in (True, False):
        idx, cnt = lsa.lsa_topk(sc, g["q_pos"], k, L, use_ws=use_ws)
        assert torch.equal(idx, res["idx"]), f"use_ws={use_ws}"
        assert torch.equal(cnt, res["count"])
    want = _flat_oracle_rows(inp, k, rows=[(0, 0), (2, 0), (3, 0), (4, 0)])
    J, out = res["idx"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for (b, i), r in want.items():
        assert np.array_equal(J[b, i], r["J"]), f"seq {b}"
        err.add(out[b, i], r["out"], (b, i))
    err.check()


@pytest.mark.parametrize("d_I", [128, 64])
def test_block_cache(lsa, d_I):
    """The block-key cache: hi, lo int8 parts with 128 * hi + lo = the block's key sum
    (lsa_block_reps, and the oracle's block_reps) and lo in [-64, 63]; a cache built in
    two partial updates over a stale buffer equals one built whole.  Block sizes on both
    sides of the per-block workgroup's threshold (32 keys), odd ones included."""
    wl = synthetic.Workload("bc", B=3, n_q=1, L=1000, q_pos0=999, H_I=4, d_I=d_I, k=16, H_q=8)
    inp, g = _inputs(wl, seed=23)
    for bs in (1, 4, 16, 31, 32, 48, 100, 128):
        full = lsa.lsa_block_cache(g["k_idx"], bs)
        reps = lsa.lsa_block_reps(g["k_idx"], bs)
        hi, lo = full[:, :, 0].long(), full[:, :, 1].long()
        assert torch.equal(128 * hi + lo, reps.long()), f"bs={bs}"
        for b in range(wl.B):
            want = oracle.block_reps(inp["k_idx"][b].numpy(), bs)
            assert np.array_equal((128 * hi + lo)[b].cpu().numpy(), want), f"bs={bs} b={b}"
        assert int(lo.min()) >= -64 and int(lo.max()) <= 63
        n = full.shape[1]
        part = torch.full_like(full, 77)
        lsa.lsa_block_cache(g["k_idx"], bs, out=part, first_block=0, n_update=n // 2)
        lsa.lsa_block_cache(g["k_idx"], bs, out=part, first_block=n // 2, n_update=n - n // 2)
        assert torch.equal(part, full), f"bs={bs}"


@pytest.mark.parametrize("case", [
    # (B, n_q, L, positions, block_size, n_keep)
    (2, 40, 3000, "random", 4, 64),     # prefill-shaped, own blocks partial and full
    (5, 1, 9000, "decode", 4, 512),     # decode-shaped, 4:1 blocks, k = 2048
    (4, 1, 40000, "decode", 4, 256),    # 10000 blocks a row: the register-resident keep
    (3, 1, 40000, "zeros", 4, 256),     # every block score 0: the lowest blocks are kept
    (1, 30, 700, "random", 16, 8),      # bigger blocks, few kept; early rows keep all
    (4, 1, 30000, "decode64", 4, 256),  # d_I = 64 and 20 heads (a partial head tile)
])
def test_forward_pooled_blocks(lsa, case):
    """Pooled blocks (two_stage = "pooled"): each query keeps its own block and the
    best n_keep - 1 earlier blocks by pooled-key score, and its list is every key of
    them it may see.  Lists, kept blocks and counts equal the oracle's (attention within
    tolerance); with a caller-built block-key cache the call skips block_reps and gives
    the same bits; where n_keep allows the token stage (n_keep <= 256), the two-stage
    path with k = n_keep * block_size gives the same bits too (its token top-k keeps
    every candidate)."""
    B, n_q, L, mode, bs, nk = case
    k = nk * bs
    H_I, d_I = (20, 64) if mode == "decode64" else (64, 128)
    wl = synthetic.Workload("pooled", B=B, n_q=n_q, L=L, q_pos0=0, H_I=H_I, d_I=d_I, k=k, H_q=16)
    if mode in ("decode", "zeros", "decode64"):
        pos = [L - 1, L - 2, 5000, 4 * nk - 1, 3][:B]
    else:
        gen = np.random.default_rng(7)
        pos = np.sort(gen.integers(0, L, (B, n_q)), axis=1)
        pos[:, 0], pos[:, 1] = 0, bs - 1
        pos = pos.reshape(-1).tolist()
    inp, g = _inputs(wl, seed=29, pos=pos)
    if mode == "zeros":
        inp["q_idx"].zero_()
        g["q_idx"].zero_()
    res = lsa.lsa_forward(g, k_top=k, two_stage="pooled", block_size=bs, n_keep=nk, attn_split=1)
    ws = lsa.lsa_forward_workspace_size(g, k, two_stage="pooled", block_size=bs, n_keep=nk)
    assert lsa.lsa_forward_stages(g, k, ws, two_stage="pooled", block_size=bs, n_keep=nk)[:3] == [
        "block_reps", "block_prefilter", "expand"]
    gc = dict(g, block_keys=lsa.lsa_block_cache(g["k_idx"], bs))
    ws = lsa.lsa_forward_workspace_size(gc, k, two_stage="pooled", block_size=bs, n_keep=nk)
    assert lsa.lsa_forward_stages(gc, k, ws, two_stage="pooled", block_size=bs, n_keep=nk)[:2] == [
        "block_prefilter", "expand"]
    res_c = lsa.lsa_forward(gc, k_top=k, two_stage="pooled", block_size=bs, n_keep=nk, attn_split=1)
    for n in ("idx", "count", "kept", "out", "lse"):
        assert torch.equal(res[n], res_c[n]), n
    if nk <= 256:
        two = lsa.lsa_forward(g, k_top=k, two_stage=True, block_size=bs, n_keep=nk, attn_split=1)
        for n in ("idx", "count", "kept", "out"):
            assert torch.equal(res[n], two[n]), n
    qi, ki, w = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["w"].numpy()
    q, kk, vv = np64(inp["q"]), np64(inp["k"]), np64(inp["v"])
    J, kept, cnt, out = res["idx"].cpu().numpy(), res["kept"].cpu().numpy(), res["count"].cpu().numpy(), np64(res["out"])
    qp = inp["q_pos"].numpy()
    rows = [(b, i) for b in range(B) for i in range(n_q)]
    if len(rows) > 12:
        rows = rows[:4] + rows[-4:] + rows[len(rows) // 2: len(rows) // 2 + 4]
    err = AttnErr()
    for b, i in rows:
        r = oracle.forward_row(qi[b, i], ki[b], w, int(qp[b, i]), k, q_row=q[b, i], k_cache=kk[b], v_cache=vv[b],
                               scale=1.0 / math.sqrt(128), two_stage=True, block_size=bs, n_keep=nk, pooled=True)
        assert np.array_equal(J[b, i], r["J"]), f"row {(b, i)}"
        assert np.array_equal(kept[b, i], r["kept"]), f"kept {(b, i)}"
        assert cnt[b, i] == r["count"]
        err.add(out[b, i], r["out"], (b, i))
    err.check()


@pytest.mark.parametrize("case", [
    # (two_stage, L, block_size, n_keep, k_top, values)
    ("pooled", 72000, 4, 300, 1200, "random"),
    ("pooled", 72000, 4, 300, 1200, "ties3"),
    ("pooled", 72000, 4, 300, 1200, "zeros"),
    ("pooled", 70002, 4, 300, 1200, "d64"),  # d_I = 64, 20 heads (a partial head tile), ragged L
])
def test_forward_block_threshold_keep(lsa, case):
    """Prefill-shaped pooled block rows over max(8 * n_keep, 16384) blocks take the
    thresholded keep: a sample of every 18th block sets each row's threshold, the block scan lists the
    blocks that reach it, and the keep comes from the list (rows whose list falls short
    or overflows are scored again into the table).  Lists, kept blocks, counts and
    outputs equal the score-table path's bit for bit with sampled thresholds, with every
    list short and with every list overflowing, and the oracle's on sampled rows.  Rows
    of at most 16384 blocks (the table) and heavily tied or all-equal scores (lists that
    overflow by themselves) mix in."""
    mode, L, bs, nk, k, vals = case
    two = "pooled" if mode == "pooled" else True
    n_q = 40
    H_I, d_I = (20, 64) if vals == "d64" else (64, 128)
    wl = synthetic.Workload("bthr", B=1, n_q=n_q, L=L, q_pos0=0, H_I=H_I, d_I=d_I, k=k, H_q=16)
    gen = np.random.default_rng(11)
    row_min = max(8 * nk, 16384)
    pos = np.sort(gen.integers(row_min * bs, L, n_q))
    pos[:4] = [0, bs * nk, row_min * bs, row_min * bs + bs]  # short rows (table), then the first list row
    pos[-1] = L - 1
    inp, g = _inputs(wl, seed=31, pos=pos.tolist())
    if vals == "zeros":
        inp["q_idx"].zero_()
    elif vals == "ties3":
        tg = torch.Generator().manual_seed(5)
        inp["q_idx"] = torch.randint(-1, 2, inp["q_idx"].shape, generator=tg).to(torch.int8)
        inp["k_idx"] = torch.randint(-1, 2, inp["k_idx"].shape, generator=tg).to(torch.int8)
    g = {n: v.to(dev()) for n, v in inp.items()}
    kw = dict(k_top=k, two_stage=two, block_size=bs, n_keep=nk, attn_split=1)
    ref = lsa.lsa_forward(g, select="table", **kw)
    for sel in ("auto", "force_short", "force_overflow"):
        res = lsa.lsa_forward(g, select=sel, **kw)
        for n in ("idx", "count", "kept", "out", "lse"):
            assert torch.equal(res[n], ref[n]), (sel, n)
    qi, ki, w = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["w"].numpy()
    q, kk, vv = np64(inp["q"]), np64(inp["k"]), np64(inp["v"])
    J, kept, out = ref["idx"].cpu().numpy(), ref["kept"].cpu().numpy(), np64(ref["out"])
    err = AttnErr()
    for i in (2, 3, n_q // 2, n_q - 1):
        r = oracle.forward_row(qi[0, i], ki[0], w, int(pos[i]), k, q_row=q[0, i], k_cache=kk[0], v_cache=vv[0],
                               scale=1.0 / math.sqrt(128), two_stage=True, block_size=bs, n_keep=nk,
                               pooled=mode == "pooled")
        assert np.array_equal(J[0, i], r["J"]), f"row {i}"
        assert np.array_equal(kept[0, i], r["kept"]), f"kept {i}"
        err.add(out[0, i], r["out"], i)
    err.check()


@pytest.mark.parametrize("mode", ["two_stage", "pooled"])
def test_forward_block_modes_short_context(lsa, mode):
    """Contexts shorter than one block (no complete block to score): every query keeps
    only its own block, so its list is keys 0..p -- decode- and prefill-shaped rows."""
    bs, nk = 64, 2
    k = nk * bs
    for B, n_q, pos in ((3, 1, [49, 0, 20]), (1, 9, list(range(0, 45, 5)))):
        wl = synthetic.Workload("short", B=B, n_q=n_q, L=50, q_pos0=0, H_I=16, d_I=64, k=k, H_q=8)
        inp, g = _inputs(wl, seed=37, pos=pos)
        res = lsa.lsa_forward(g, k_top=k, two_stage="pooled" if mode == "pooled" else True, block_size=bs,
                              n_keep=nk, attn_split=1)
        J = res["idx"].cpu().numpy()
        for b in range(B):
            for i in range(n_q):
                p = int(inp["q_pos"][b, i])
                want = np.concatenate([np.arange(p + 1), np.full(k - p - 1, -1)])
                assert np.array_equal(J[b, i], want), f"{mode} {(b, i)}"
                assert int(res["count"][b, i]) == p + 1


def _map_pages(J, page_table, page_size):
    """Logical keys [B, n_q, k] (or -1) -> pool rows through page_table [B, max_pages]."""
    J = J.long()
    pt = page_table.long()
    B, n_q, k = J.shape
    Jc = J.clamp(min=0)
    rows = torch.gather(pt, 1, (Jc // page_size).reshape(B, -1)).reshape(B, n_q, k) * page_size + Jc % page_size
    return torch.where(J >= 0, rows, torch.full_like(J, -1))


@pytest.mark.parametrize("page_size,H_I,d_I", [(64, 64, 128), (256, 64, 128), (128, 20, 64)])
def test_forward_decode_paged(lsa, page_size, H_I, d_I):
    """Paged caches (decode): k_idx / k / v are pools shared by the sequences, each
    sequence reaching its keys through a page table (pages scattered over the pool,
    spare pages between them).  The lists name pool rows: they equal the contiguous
    call's lists mapped through the page table, counts equal, outputs and LSE equal
    bit for bit; the oracle's paged definition agrees on sampled rows.  Sequences of
    different lengths share the call, rows of at most k keys included."""
    L, k = 40000, 1024
    pos = [39999, 30000, 1023, 500, 33333, 39998, 4095]
    wl = synthetic.Workload("paged", B=len(pos), n_q=1, L=L, q_pos0=0, H_I=H_I, d_I=d_I, k=k, H_q=16)
    inp, g = _inputs(wl, seed=13, pos=pos)
    ref = lsa.lsa_forward(g, k_top=k)
    pg = synthetic.paged_pool(g, page_size, spare_pages=37, seed=3)
    ws_bytes = lsa.lsa_forward_workspace_size(pg, k)
    assert lsa.lsa_forward_stages(pg, k, ws_bytes) == ["index_select", "topk", "sparse_attn"]
    res = lsa.lsa_forward(pg, k_top=k)
    torch.cuda.synchronize()
    assert torch.equal(res["idx"].long(), _map_pages(ref["idx"], pg["page_table"], page_size))
    assert torch.equal(res["count"], ref["count"])
    assert torch.equal(res["out"], ref["out"])
    assert torch.equal(res["lse"], ref["lse"])
    # the oracle over the pool itself
    pt = pg["page_table"].cpu().numpy()
    pki, pk, pv = pg["k_idx"].cpu().numpy(), np64(pg["k"].cpu()), np64(pg["v"].cpu())
    qi, w, q = inp["q_idx"].numpy(), inp["w"].numpy(), np64(inp["q"])
    J, out = res["idx"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for b in (0, 3, 6):
        r = oracle.forward_row_paged(qi[b, 0], pki, w, pos[b], k, pt[b], page_size, q_row=q[b, 0],
                                     k_pool=pk, v_pool=pv, scale=1.0 / math.sqrt(128))
        assert np.array_equal(J[b, 0], r["J"]), f"seq {b}"
        err.add(out[b, 0], r["out"], b)
    err.check()


@pytest.mark.parametrize("page_size", [64, 256])
def test_forward_prefill_paged(lsa, page_size):
    """Paged caches in prefill chunks (the flat indexer reads keys through the page
    table): every selection mode -- thresholded lists, forced fall-backs, the score
    table -- gives the contiguous call's lists mapped through the page table, its counts
    and outputs bit for bit; rows up to 4096 keys (the table) and a short last chunk of
    two queries (the decode selection) mix in."""
    k = 512
    wl = synthetic.Workload("pgpre", B=2, n_q=98, L=24000, q_pos0=0, H_I=64, d_I=128, k=k, H_q=16)
    pos = np.linspace(0, 23999, 98).astype(np.int64)
    pos[:6] = [0, 300, 511, 512, 4095, 4096]
    _, g = _inputs(wl, seed=31, pos=np.tile(pos, 2))
    pg = synthetic.paged_pool(g, page_size, spare_pages=29, seed=7)
    for mode in ("auto", "table", "force_short", "force_overflow"):
        ref = lsa.lsa_forward(g, k_top=k, select=mode, attn_split=1, chunk_rows=48)
        res = lsa.lsa_forward(pg, k_top=k, select=mode, attn_split=1, chunk_rows=48)
        torch.cuda.synchronize()
        assert torch.equal(res["idx"].long(), _map_pages(ref["idx"], pg["page_table"], page_size)), mode
        assert torch.equal(res["count"], ref["count"]), mode
        assert torch.equal(res["out"], ref["out"]), mode
        assert torch.equal(res["lse"], ref["lse"]), mode


@pytest.mark.parametrize("mode,B,n_q,L,bs,nk,k,P", [
    ("two_stage", 5, 1, 20480, 128, 64, 2048, 64),   # decode rows, the one-kernel token stage
    ("two_stage", 2, 40, 9024, 128, 20, 600, 64),    # prefill rows; own blocks run past the last page
    ("two_stage", 2, 30, 3072, 16, 6, 40, 64),       # blocks of 16: slots looked up one by one
    ("pooled", 5, 1, 9216, 4, 512, 2048, 64),        # decode rows, 4:1 pooled keys
    ("pooled", 2, 40, 3072, 4, 64, 256, 256),        # prefill rows
])
def test_forward_block_modes_paged(lsa, mode, B, n_q, L, bs, nk, k, P):
    """Block modes over paged caches: the block-key cache built through the page table
    equals the contiguous one; kept blocks, counts, outputs and LSE equal the
    contiguous call's bit for bit and the lists are its lists mapped through the page
    table (also with the caller's paged block-key cache); the oracle's paged definition
    agrees on sampled rows."""
    two = "pooled" if mode == "pooled" else True
    wl = synthetic.Workload("pgblk", B=B, n_q=n_q, L=L, q_pos0=0, H_I=64, d_I=128, k=k, H_q=16)
    if n_q == 1:
        pos = [L - 1, L - 2, L // 2 + 3, 4 * nk * bs // 4 - 1, 3][:B]
    else:
        pos = np.sort(np.random.default_rng(17).integers(0, L, (B, n_q)), axis=1)
        pos[:, 0], pos[:, 1], pos[:, -1] = 0, bs - 1, L - 1
        pos = pos.reshape(-1).tolist()
    inp, g = _inputs(wl, seed=41, pos=pos)
    ref = lsa.lsa_forward(g, k_top=k, two_stage=two, block_size=bs, n_keep=nk, attn_split=1)
    pg = synthetic.paged_pool(g, P, spare_pages=23, seed=9)
    res = lsa.lsa_forward(pg, k_top=k, two_stage=two, block_size=bs, n_keep=nk, attn_split=1)
    torch.cuda.synchronize()
    assert torch.equal(res["kept"], ref["kept"])
    assert torch.equal(res["idx"].long(), _map_pages(ref["idx"], pg["page_table"], P))
    for name in ("count", "out", "lse"):
        assert torch.equal(res[name], ref[name]), name
    # the block-key cache through the page table, and the call that takes it
    bk = lsa.lsa_block_cache(pg["k_idx"], bs, page_table=pg["page_table"], page_size=P)
    assert torch.equal(bk[:, : L // bs], lsa.lsa_block_cache(g["k_idx"], bs))
    res_c = lsa.lsa_forward(dict(pg, block_keys=bk), k_top=k, two_stage=two, block_size=bs, n_keep=nk, attn_split=1)
    torch.cuda.synchronize()
    for name in ("idx", "count", "kept", "out", "lse"):
        assert torch.equal(res_c[name], res[name]), name
    # the oracle over the pool itself
    pt = pg["page_table"].cpu().numpy()
    pki, pk, pv = pg["k_idx"].cpu().numpy(), np64(pg["k"].cpu()), np64(pg["v"].cpu())
    qi, w, q = inp["q_idx"].numpy(), inp["w"].numpy(), np64(inp["q"])
    J, kept, out = res["idx"].cpu().numpy(), res["kept"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for b, i in [(0, 0), (B - 1, n_q - 1), (B // 2, n_q // 2)]:
        p = int(inp["q_pos"][b, i])
        r = oracle.forward_row_paged(qi[b, i], pki, w, p, k, pt[b], P, q_row=q[b, i], k_pool=pk, v_pool=pv,
                                     scale=1.0 / math.sqrt(128), two_stage=True, block_size=bs, n_keep=nk,
                                     pooled=mode == "pooled")
        assert np.array_equal(kept[b, i], r["kept"]), (b, i)
        assert np.array_equal(J[b, i], r["J"]), (b, i)
        err.add(out[b, i], r["out"], (b, i))
    err.check()


def test_forward_decode_paged_graph_replay(lsa):
    """A paged decode step captured once in a HIP graph (one graph per range of context
    lengths: the page-table width fixes L_max and so every launch shape) replays for
    new positions and new page tables written into the captured inputs; every replay
    equals an eager call on the same inputs, bit for bit."""
    P, k, L = 64, 512, 20000
    pos = [19999, 12000, 511, 7000]
    wl = synthetic.Workload("pgraph", B=len(pos), n_q=1, L=L, q_pos0=0, H_I=64, d_I=128, k=k, H_q=16)
    _, g = _inputs(wl, seed=17, pos=pos)
    pg = synthetic.paged_pool(g, P, spare_pages=64, seed=5)
    ws = torch.empty((max(lsa.lsa_forward_workspace_size(pg, k), 16),), dtype=torch.uint8, device=dev())
    B = len(pos)
    out = {"idx": torch.empty((B, 1, k), dtype=torch.int32, device=dev()),
           "count": torch.empty((B, 1), dtype=torch.int32, device=dev()),
           "out": torch.empty_like(pg["q"]),
           "lse": torch.empty((B, 1, 16), dtype=torch.float32, device=dev())}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lsa.lsa_forward(pg, k_top=k, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lsa.lsa_forward(pg, k_top=k, out=out, ws=ws)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(99)
    n_pool = pg["k_idx"].shape[0] // P
    for trial in range(3):
        new_pos = torch.randint(0, L, (B, 1), generator=gen, dtype=torch.int32)
        new_pt = torch.randperm(n_pool, generator=gen)[: pg["page_table"].numel()].to(torch.int32)
        pg["q_pos"].copy_(new_pos.to(dev()))
        pg["page_table"].copy_(new_pt.view_as(pg["page_table"]).to(dev()))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {n: t.clone() for n, t in out.items()}
        want = lsa.lsa_forward(pg, k_top=k)
        torch.cuda.synchronize()
        for n in ("idx", "count", "out", "lse"):
            assert torch.equal(got[n], want[n]), f"replay {trial}: {n}"


@pytest.mark.parametrize("kind", ["one_span_distinct", "whole_span_equal", "two_spans_ties", "all_equal",
                                  "spread_ties"])
def test_forward_decode_fused_selection_concentrated(lsa, kind):
    """Decode rows with awkward score distributions for the indexer's span lists
    (19 spans of <= 2112 keys per row here, lists of >= min(span, k) entries and at
    most 2k): the top-k concentrated in about one span; a run of 3616 identical keys
    that covers whole spans (such a span's list would overflow: it writes its table
    slice, the row stays on the list path); ties in two spans; all scores equal (the
    cut bin overflows the LDS list: the row's table is completed from lists and
    slices, exact radix fallback, table slices and whole-span lists mixed); ~5000
    ties spread over every span (the same fallback from lists only) -- still bit for
    bit the separate calls' lists and the oracle's."""
    L, k = 40000, 1024
    pos = [39999, 39000, 35000, 20000]
    wl = synthetic.Workload("deccon", B=len(pos), n_q=1, L=L, q_pos0=0, H_I=64, d_I=128, k=k, H_q=16)
    inp, _ = _inputs(wl, seed=12, pos=pos)
    q0 = inp["q_idx"][:, 0, 0, :].clone()           # head 0 of each query: keys aligned with it score high
    gen = torch.Generator().manual_seed(3)
    for b in range(wl.B):
        if kind == "one_span_distinct":
            lo, hi = 16384, 18432                     # 2048 keys: about one span
            noise = torch.randint(-3, 4, (hi - lo, 128), generator=gen, dtype=torch.int64)
            inp["k_idx"][b, lo:hi] = (q0[b].to(torch.int64) + noise).clamp(-128, 127).to(torch.int8)
        elif kind == "whole_span_equal":
            lo, hi = 16384, 20000                     # 3616 identical keys (ties), whole spans
            inp["k_idx"][b, lo:hi] = q0[b]
        elif kind == "two_spans_ties":
            for lo, hi in ((2048, 2600), (10240, 10900)):   # two spans, ties inside each
                inp["k_idx"][b, lo:hi] = q0[b]
        elif kind == "all_equal":
            inp["q_idx"][b] = 0                       # every score 0: the cut bin holds the whole row
        else:
            inp["k_idx"][b, 0:L:8] = q0[b]            # ~5000 ties spread over every span
    g = {kk: v.to(dev()) for kk, v in inp.items()}
    assert lsa.lsa_forward_stages(g, k, lsa.lsa_forward_workspace_size(g, k))[0] == "index_select"
    res = lsa.lsa_forward(g, k_top=k)
    ld = ((L + 63) // 64) * 64
    sc = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"], ld=ld)
    for use_ws in (True, False):
        idx, cnt = lsa.lsa_topk(sc, g["q_pos"], k, L, use_ws=use_ws)
        assert torch.equal(idx, res["idx"]), f"{kind} use_ws={use_ws}"
        assert torch.equal(cnt, res["count"])
    want = _flat_oracle_rows(inp, k, with_attn=False, rows=[(0, 0), (3, 0)])
    J = res["idx"].cpu().numpy()
    for (b, i), r in want.items():
        assert np.array_equal(J[b, i], r["J"]), f"{kind} seq {b}"


@pytest.mark.parametrize("T,bs,n_keep,k", [(4096, 128, 8, 256), (2048, 16, 6, 40), (20000, 128, 64, 2048),
                                           (20000, 128, 100, 2048), (5000, 64, 20, 300), (9000, 64, 150, 1000)])
def test_forward_two_stage_small(lsa, T, bs, n_keep, k):
    """Two-stage lsa_forward against the oracle, and bit for bit against the separate calls
    (block prefilter, kept-slot scores, score-table top-k): with at most 8192 kept slots
    the forward scores and selects in one kernel, above that through the score table."""
    n_q = 64
    wl = synthetic.Workload("ts", B=1, n_q=n_q, L=T, q_pos0=T - n_q, H_I=64, d_I=128, k=k, H_q=16,
                            two_stage=True, block_size=bs, n_keep=n_keep)
    inp, g = _inputs(wl, seed=6)
    res = lsa.lsa_forward(g, k_top=k, two_stage=True, block_size=bs, n_keep=n_keep)
    kept_g = lsa.lsa_block_prefilter(g["q_idx"], lsa.lsa_block_reps(g["k_idx"], bs), g["w"], g["q_pos"], bs, n_keep)
    sc = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"], kept_blocks=kept_g, block_size=bs,
                              n_keep=n_keep)
    idx2, cnt2 = lsa.lsa_topk(sc, g["q_pos"], k, T, kept_blocks=kept_g, block_size=bs)
    assert torch.equal(kept_g, res["kept"])
    assert torch.equal(idx2, res["idx"])
    assert torch.equal(cnt2, res["count"])
    qi, ki, w = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["w"].numpy()
    q, kk, vv = np64(inp["q"]), np64(inp["k"]), np64(inp["v"])
    reps = oracle.block_reps(ki[0], bs)
    J, kept, out = res["idx"].cpu().numpy(), res["kept"].cpu().numpy(), np64(res["out"])
    err = AttnErr()
    for i in range(n_q):
        p = int(inp["q_pos"][0, i])
        r = oracle.forward_row(qi[0, i], ki[0], w, p, k, q_row=q[0, i], k_cache=kk[0], v_cache=vv[0],
                               scale=1 / math.sqrt(128), two_stage=True, block_size=bs, n_keep=n_keep, reps=reps)
        assert np.array_equal(kept[0, i], r["kept"]), f"kept row {i}"
        assert np.array_equal(J[0, i], r["J"]), f"J row {i}"
        err.add(out[0, i], r["out"], i)
    err.check()


def test_forward_two_stage_without_key_copy(lsa):
    """A prefill-shaped two-stage forward whose workspace cannot hold the token stage's
    interleaved key copy reads the key rows instead (in chunks of the rows that fit): the
    same kept blocks, lists, counts and outputs bit for bit."""
    T, bs, n_keep, k, n_q = 20000, 128, 64, 2048, 64
    wl = synthetic.Workload("ts_nocopy", B=1, n_q=n_q, L=T, q_pos0=T - n_q, H_I=64, d_I=128, k=k, H_q=16,
                            two_stage=True, block_size=bs, n_keep=n_keep)
    inp, g = _inputs(wl, seed=8)
    ref = lsa.lsa_forward(g, k_top=k, two_stage=True, block_size=bs, n_keep=n_keep)
    small = (T + 63) // 64 * 64 * 128 - (1 << 16)
    rows, split = lsa.lsa_forward_plan(g, k, small, two_stage=True, block_size=bs, n_keep=n_keep)
    assert 0 < rows < n_q and split == lsa.lsa_forward_plan(g, k, 1 << 30, two_stage=True, block_size=bs,
                                                             n_keep=n_keep)[1]
    ws = torch.empty((small,), dtype=torch.uint8, device=dev())
    res = lsa.lsa_forward(g, k_top=k, two_stage=True, block_size=bs, n_keep=n_keep, ws=ws)
    torch.cuda.synchronize()
    for name in ("kept", "idx", "count", "out", "lse"):
        assert torch.equal(res[name], ref[name]), name


def test_forward_two_stage_reduces_to_flat(lsa):
    """When every causal block is kept (own < n_keep) the two-stage lists equal the flat ones."""
    wl = synthetic.Workload("red", B=1, n_q=128, L=1024, q_pos0=896, H_I=64, d_I=128, k=200, H_q=16)
    _, g = _inputs(wl, seed=8)
    flat = lsa.lsa_forward(g, k_top=wl.k)
    two = lsa.lsa_forward(g, k_top=wl.k, two_stage=True, block_size=128, n_keep=64)
    assert torch.equal(flat["idx"], two["idx"])
    assert torch.equal(flat["out"], two["out"])


def test_edge_rows_and_errors(lsa):
    """Negative positions give empty rows; invalid arguments return errors, launch nothing."""
    wl = synthetic.Workload("e", B=1, n_q=4, L=100, q_pos0=0, H_I=16, d_I=64, k=8, H_q=8)
    inp, g = _inputs(wl, seed=9, pos=[-1, 0, 3, 99])
    res = lsa.lsa_forward(g, k_top=8)
    J = res["idx"].cpu().numpy()[0]
    assert list(J[0]) == [-1] * 8
    assert list(J[1]) == [0] + [-1] * 7
    assert list(J[2]) == [0, 1, 2, 3] + [-1] * 4
    assert torch.all(res["out"][0, 0].cpu() == 0)
    assert torch.all(torch.isneginf(res["lse"][0, 0].cpu()))
    with pytest.raises(lsa.LsaError):
        lsa.lsa_topk(torch.zeros((1, 2, 10), dtype=torch.int32, device=dev()),
                     torch.zeros((1, 2), dtype=torch.int32, device=dev()), 5000, 10)   # k > 4096
    with pytest.raises(lsa.LsaError):
        bad = dict(g)
        bad["q"] = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16, device=dev())   # d != 128
        lsa.lsa_sparse_attn(bad["q"], g["k"][..., :64].contiguous(), g["v"][..., :64].contiguous(),
                            res["idx"])
