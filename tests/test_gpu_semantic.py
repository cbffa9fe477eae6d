"""Flat semantic search on the GPU against the CPU oracle: the bucket cache (centroid
bits, key tables, offsets) and the index lists bit for bit, attention over the lists
within tolerance, at small sizes spanning several blocks and ragged tails and on
sampled rows of the full-size workloads."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import AttnErr, dev, np64

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module")
def lsa():
    import learned_top_sparse_amd as m
    m.lib()
    return m


def _f32(t):
    return t.detach().float().cpu().numpy().astype(np.float32)


def _gpu_cache_np(cache, b):
    """The GPU cache of sequence b in the oracle's layout: centroids [NB, m, 64]."""
    c = cache["centroids"][b].float().cpu().numpy()             # [NB, 8, 64, 8]
    m = cache["offsets"].shape[-1] - 1
    cent = c.transpose(0, 2, 1, 3).reshape(c.shape[0], 64, 64)[:, :m]
    return cent, cache["table"][b].cpu().numpy(), cache["offsets"][b].cpu().numpy()


def _oracle_cache(k_sem_b, prm, n_blocks=None):
    n_cluster, n_pool, n_bavg, n_bmax = prm
    return oracle.bucket_cache(_f32(k_sem_b), n_cluster, n_pool, n_bavg, n_bmax, n_blocks=n_blocks)


def _check_cache(cache, k_sem, prm, blocks=None):
    B = k_sem.shape[0]
    for b in range(B):
        cent, table, offs = _gpu_cache_np(cache, b)
        NB = table.shape[0]
        want = _oracle_cache(k_sem[b], prm, n_blocks=NB)
        sel = range(NB) if blocks is None else blocks
        for t in sel:
            assert np.array_equal(offs[t], want["offsets"][t]), f"offsets b={b} block={t}"
            assert np.array_equal(table[t], want["table"][t]), f"table b={b} block={t}"
            assert np.array_equal(cent[t], want["centroids"][t]), f"centroids b={b} block={t}"
        # unused slots of the centroid layout stay zero
        m = offs.shape[-1] - 1
        full = cache["centroids"][b].float().cpu().numpy().transpose(0, 2, 1, 3).reshape(NB, 64, 64)
        assert not full[:, m:].any()
    return want


PARAMS = [(512, 4, 8, 32), (256, 2, 4, 16), (128, 1, 2, 8), (512, 8, 16, 64), (64, 2, 4, 8)]


@pytest.mark.parametrize("prm", PARAMS, ids=lambda p: "c%d_p%d_a%d_x%d" % p)
def test_cluster_matches_oracle(lsa, prm):
    n_cluster = prm[0]
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=2, L=3 * n_cluster + 77, q_pos0=3 * n_cluster + 76)
    inp = synthetic.semantic_inputs(wl, dev(), seed=3)
    print(f"[cluster {prm}]", flush=True)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    torch.cuda.synchronize()
    assert cache["table"].shape[1] == wl.L // n_cluster
    _check_cache(cache, inp["k_sem"], prm)


def test_cluster_degenerate_keys(lsa):
    """All-zero keys (zero pool keys: every cost 0, ties everywhere) and identical keys."""
    prm = (512, 4, 8, 32)
    k = torch.zeros((2, 1024, 64), dtype=torch.bfloat16, device=dev())
    k[1] = torch.randn(64, device=dev()).to(torch.bfloat16)     # every key the same
    k[0, 512:] = torch.randn((512, 64), device=dev()).to(torch.bfloat16)
    cache = lsa.lsa_semantic_cache(k, *prm)
    torch.cuda.synchronize()
    _check_cache(cache, k, prm)


def test_cluster_incremental(lsa):
    """Clustering blocks one at a time into a cache sized for more gives the same cache."""
    prm = (512, 4, 8, 32)
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=3, L=4 * 512, q_pos0=4 * 512 - 1)
    inp = synthetic.semantic_inputs(wl, dev(), seed=4)
    full = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    inc = lsa.lsa_semantic_cache(inp["k_sem"][:, :512].contiguous(), *prm, n_blocks=4)
    for t in range(1, 4):
        inc = lsa.lsa_semantic_cache(inp["k_sem"], cache=inc, first_block=t, n_update=1)
    torch.cuda.synchronize()
    for name in ("centroids", "table", "offsets"):
        assert torch.equal(full[name], inc[name]), name


def _select_case(lsa, wl, prm, positions, k, p_top, n_sink, n_w, seed, ws_bytes=None):
    inp = synthetic.semantic_inputs(wl, dev(), seed=seed)
    B = wl.B
    q_pos = torch.tensor(positions, dtype=torch.int32, device=dev()).view(B, -1).contiguous()
    q = inp["q_sem"][:, :1].expand(B, q_pos.shape[1], 64).contiguous()
    q = q + torch.randn(q.shape, device=dev(), generator=torch.Generator(dev()).manual_seed(seed)).to(q.dtype)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    idx, cnt = lsa.lsa_semantic_select(q, q_pos, cache, k, p_top, n_sink, n_w, ws_bytes=ws_bytes)
    torch.cuda.synchronize()
    return inp, q, q_pos, cache, idx, cnt


@pytest.mark.parametrize("prm,k,p_top,n_sink,n_w", [
    ((512, 4, 8, 32), 300, 80, 4, 512),
    ((512, 4, 8, 32), 2048, 512, 4, 512),
    ((256, 2, 4, 16), 100, 64, 0, 300),
    ((128, 1, 2, 8), 77, 2048, 9, 1),
    ((512, 4, 8, 32), 500, 128, 4, 1),
    ((512, 4, 8, 128), 300, 80, 4, 512),   # buckets of up to 128 keys: the streaming selection
])
def test_select_matches_oracle(lsa, prm, k, p_top, n_sink, n_w):
    n_c = prm[0]
    L = 9 * n_c + 5
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=2, L=L, q_pos0=L - 1)
    positions = [[L - 1, n_c - 1, n_c, 2 * n_c + 3, 5 * n_c - 1, 0, -1, 8 * n_c + 100],
                 [3, L - 2, 7 * n_c, n_c + 1, 4 * n_c + 17, 6 * n_c, 2 * n_c - 1, L - 1]]
    inp, q, q_pos, cache, idx, cnt = _select_case(lsa, wl, prm, positions, k, p_top, n_sink, n_w, seed=5)
    for b in range(2):
        oc = _oracle_cache(inp["k_sem"][b], prm, n_blocks=cache["table"].shape[1])
        for i, p in enumerate(positions[b]):
            r = oracle.semantic_select_row(_f32(q[b, i]), oc, p, k, p_top, n_sink, n_w)
            assert np.array_equal(idx[b, i].cpu().numpy(), r["J"]), f"b={b} p={p}"
            assert int(cnt[b, i]) == r["count"], f"count b={b} p={p}"


def test_select_threshold_modes(lsa):
    """Decode rows (one query per sequence) through the threshold list: a sampled
    threshold, the buckets at or above it listed by the scan, the list ranked; rows whose
    list falls short or overflows rank their whole row.  Rows of 5120 and 4480 buckets
    (listed), of 3840 (at most the list: every bucket listed), inside the first block and
    padding.  Every mode -- the list, the whole row, and both forced fall-backs -- gives
    the same lists bit for bit, paged storage the same lists mapped to pool rows, and
    sampled rows equal the oracle's."""
    prm = (512, 4, 8, 32)
    L = 80 * 512
    P = 64
    positions = [L - 1, 70 * 512 + 5, 60 * 512, 300, -1, 79 * 512 + 17]
    B = len(positions)
    wl = synthetic.Workload("sem_thr", B=B, n_q=1, L=L, q_pos0=L - 1, H_I=1, d_I=64, k=2048, H_q=16, semantic=True,
                            p_top=512, n_sink=4)
    inp = synthetic.semantic_inputs(wl, dev(), seed=31)
    q_pos = torch.tensor(positions, dtype=torch.int32, device=dev()).view(B, 1)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    res = {}
    for mode in ("threshold", "row", "force_short", "force_overflow"):
        print(f"[threshold modes: {mode}]", flush=True)
        res[mode] = lsa.lsa_semantic_select(inp["q_sem"], q_pos, cache, 2048, 512, 4, 512, select=mode)
    torch.cuda.synchronize()
    for mode in ("threshold", "force_short", "force_overflow"):
        assert torch.equal(res[mode][0], res["row"][0]), mode
        assert torch.equal(res[mode][1], res["row"][1]), mode
    # paged storage: the same lists as pool rows
    NB, max_pages = L // 512, L // P
    gen = torch.Generator().manual_seed(32)
    n_pages = B * max_pages + 9
    pt = torch.randperm(n_pages, generator=gen)[: B * max_pages].view(B, max_pages).to(torch.int32).to(dev())
    n_bslots = B * NB + 3
    bt = torch.randperm(n_bslots, generator=gen)[: B * NB].view(B, NB).to(torch.int32).to(dev())
    paged = {"block_table": bt, "page_table": pt, "page_size": P, "n_slots": n_pages * P}
    cache_p = lsa.lsa_semantic_cache(_to_pool(inp["k_sem"], pt, P, n_pages, 4), *prm, paged=paged, n_bslots=n_bslots)
    idx_p, cnt_p = lsa.lsa_semantic_select(inp["q_sem"], q_pos, cache_p, 2048, 512, 4, 512, paged=paged,
                                           select="threshold")
    idx = res["threshold"][0]
    mapped = torch.where(idx >= 0, pt.long().gather(1, (idx.clamp(min=0) // P).view(B, -1)).view_as(idx) * P
                         + idx.clamp(min=0) % P, torch.full_like(idx, -1).long()).to(torch.int32)
    assert torch.equal(idx_p, mapped) and torch.equal(cnt_p, res["threshold"][1])
    for b in (0, 2, 3, 5):
        oc = _oracle_cache(inp["k_sem"][b], prm, n_blocks=NB)
        r = oracle.semantic_select_row(_f32(inp["q_sem"][b, 0]), oc, positions[b], 2048, 512, 4, 512)
        assert np.array_equal(idx[b, 0].cpu().numpy(), r["J"]), f"b={b}"
        assert int(res["threshold"][1][b, 0]) == r["count"]


@pytest.mark.slow
def test_select_threshold_long_rows(lsa):
    """Decode rows of 70400 buckets (1100 blocks) through the threshold list, with a
    sample of N / 8 buckets: the same lists as the whole-row ranking and both forced
    fall-backs, bit for bit."""
    prm = (512, 4, 8, 32)
    L = 1100 * 512 + 7
    positions = [L - 1, L - 5000, 900 * 512 + 11]
    B = len(positions)
    wl = synthetic.Workload("sem_thr_long", B=B, n_q=1, L=L, q_pos0=L - 1, H_I=1, d_I=64, k=2048, H_q=16,
                            semantic=True, p_top=512, n_sink=4)
    inp = synthetic.semantic_inputs(wl, dev(), seed=33)
    q_pos = torch.tensor(positions, dtype=torch.int32, device=dev()).view(B, 1)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    res = {mode: lsa.lsa_semantic_select(inp["q_sem"], q_pos, cache, 2048, 512, 4, 512, select=mode)
           for mode in ("threshold", "row", "force_short", "force_overflow")}
    torch.cuda.synchronize()
    for mode in ("threshold", "force_short", "force_overflow"):
        assert torch.equal(res[mode][0], res["row"][0]), mode
        assert torch.equal(res[mode][1], res["row"][1]), mode


def test_select_empty_cache(lsa):
    """A cache of no blocks (contexts shorter than one cluster block): every list is the
    sink and the window, as the oracle's."""
    prm = (512, 4, 8, 32)
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=2, L=500, q_pos0=499)
    inp = synthetic.semantic_inputs(wl, dev(), seed=12)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    assert cache["table"].shape[1] == 0
    q_pos = torch.tensor([[499, 3], [0, -1]], dtype=torch.int32, device=dev())
    q = inp["q_sem"].expand(2, 2, 64).contiguous()
    idx, cnt = lsa.lsa_semantic_select(q, q_pos, cache, 100, 16, 4, 512)
    torch.cuda.synchronize()
    oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=0)
    for b in range(2):
        for i in range(2):
            r = oracle.semantic_select_row(_f32(q[b, i]), oc, int(q_pos[b, i]), 100, 16, 4, 512)
            assert np.array_equal(idx[b, i].cpu().numpy(), r["J"]) and int(cnt[b, i]) == r["count"]


def test_select_in_chunks(lsa):
    """A workspace for one query per sequence: the call runs in chunks, same lists."""
    prm = (512, 4, 8, 32)
    L = 6 * 512
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=2, L=L, q_pos0=L - 1)
    positions = [[L - 1 - 37 * i for i in range(20)], [512 + 97 * i for i in range(20)]]
    inp, q, q_pos, cache, idx, cnt = _select_case(lsa, wl, prm, positions, 200, 64, 4, 512, seed=6)
    row = 64 * 4 + ((cache["table"].shape[1] * 64 + 3) // 4 * 4) * 4
    idx2, cnt2 = lsa.lsa_semantic_select(q, q_pos, cache, 200, 64, 4, 512, ws_bytes=2 * row * 3)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)


def test_semantic_forward_small(lsa):
    """Selection and attention together on a causal chunk against the oracle."""
    prm = (512, 4, 8, 32)
    wl = synthetic.Workload("sem_small", B=2, n_q=64, L=5 * 512 + 40, q_pos0=5 * 512 - 24, H_I=1, d_I=64,
                            k=256, H_q=8, d=128, semantic=True, p_top=64, n_sink=4)
    g = synthetic.make_inputs(wl.replace(d_I=64), dev())
    g.update(synthetic.semantic_inputs(wl, dev(), seed=7))
    cache = lsa.lsa_semantic_cache(g["k_sem"], *prm)
    res = lsa.lsa_semantic_forward(g, cache, wl.k, wl.p_top, wl.n_sink, prm[0])
    torch.cuda.synchronize()
    err = AttnErr()
    for b in range(2):
        oc = _oracle_cache(g["k_sem"][b], prm, n_blocks=cache["table"].shape[1])
        for i in range(0, 64, 5):
            p = int(g["q_pos"][b, i])
            r = oracle.semantic_forward_row(_f32(g["q_sem"][b, i]), oc, p, wl.k, wl.p_top, wl.n_sink, prm[0],
                                            q_row=np64(g["q"][b, i]), k_cache=np64(g["k"][b]),
                                            v_cache=np64(g["v"][b]), scale=wl.scale)
            assert np.array_equal(res["idx"][b, i].cpu().numpy(), r["J"]), f"b={b} i={i}"
            assert int(res["count"][b, i]) == r["count"]
            err.add(np64(res["out"][b, i]), r["out"], (b, i))
    err.check()


def test_select_many_rows(lsa):
    """A prefill chunk of 600 queries (enough rows for the two-workgroups-per-CU
    selection): sampled rows, first and last included, bit for bit."""
    prm = (512, 4, 8, 32)
    L = 12 * 512 + 30
    wl = synthetic.Workload("sem_chunk", B=1, n_q=600, L=L, q_pos0=L - 600, H_I=1, d_I=64, k=300, H_q=16,
                            semantic=True, p_top=64, n_sink=4)
    inp = synthetic.semantic_inputs(wl, dev(), seed=10)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    idx, cnt = lsa.lsa_semantic_select(inp["q_sem"], inp["q_pos"], cache, wl.k, wl.p_top, wl.n_sink, prm[0])
    torch.cuda.synchronize()
    oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=cache["table"].shape[1])
    for i in [0, 1, 77, 150, 299, 300, 451, 598, 599] + list(range(5, 600, 41)):
        p = int(inp["q_pos"][0, i])
        r = oracle.semantic_select_row(_f32(inp["q_sem"][0, i]), oc, p, wl.k, wl.p_top, wl.n_sink, prm[0])
        assert np.array_equal(idx[0, i].cpu().numpy(), r["J"]), f"i={i} p={p}"
        assert int(cnt[0, i]) == r["count"]


@pytest.mark.slow
def test_prefill_128k_lsa_sampled(lsa):
    """The prefill workload at full size (8192 queries of a 128K context) as the benchmark
    runs it: the cache of the blocks before the chunk, then the chunk's own 16 blocks
    clustered into it, then the selection; sampled rows against the oracle's clustering."""
    wl = synthetic.WORKLOADS["prefill_128k_lsa"]
    prm = (wl.n_cluster, wl.n_pool, wl.n_bavg, wl.n_bmax)
    inp = synthetic.semantic_inputs(wl, dev())
    first = wl.q_pos0 // wl.n_cluster
    cache = lsa.lsa_semantic_cache(inp["k_sem"][:, :wl.q_pos0].contiguous(), *prm, n_blocks=wl.L // wl.n_cluster)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], cache=cache, first_block=first,
                                   n_update=wl.L // wl.n_cluster - first)
    idx, cnt = lsa.lsa_semantic_select(inp["q_sem"], inp["q_pos"], cache, wl.k, wl.p_top, wl.n_sink, wl.n_cluster)
    torch.cuda.synchronize()
    print("[prefill_128k_lsa] oracle cache", flush=True)
    oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=cache["table"].shape[1])
    for i in (0, 1, 511, 512, 4000, 8190, 8191):
        p = int(inp["q_pos"][0, i])
        r = oracle.semantic_select_row(_f32(inp["q_sem"][0, i]), oc, p, wl.k, wl.p_top, wl.n_sink, wl.n_cluster)
        assert np.array_equal(idx[0, i].cpu().numpy(), r["J"]), f"i={i} p={p}"
        assert int(cnt[0, i]) == r["count"]


@pytest.mark.slow
def test_select_long_rows(lsa):
    """Rows of more buckets than the registers hold (37440 > 32768): spans of 16384
    buckets as workgroups of their own (few rows), their candidates merged, bit for
    bit; and buckets of 16 keys (key positions beyond the smaller bitmaps)."""
    for prm, L in (((512, 4, 8, 32), 585 * 512 + 3), ((512, 4, 16, 32), 300 * 512 + 9)):
        wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=1, L=L, q_pos0=L - 1)
        positions = [[L - 1, L - 600, 200 * 512 + 5, 3 * 512]]
        print(f"[long rows {prm} L={L}]", flush=True)
        inp, q, q_pos, cache, idx, cnt = _select_case(lsa, wl, prm, positions, 2048, 512, 4, 512, seed=8)
        oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=cache["table"].shape[1])
        for i, p in enumerate(positions[0]):
            r = oracle.semantic_select_row(_f32(q[0, i]), oc, p, 2048, 512, 4, 512)
            assert np.array_equal(idx[0, i].cpu().numpy(), r["J"]), f"p={p}"
            assert int(cnt[0, i]) == r["count"]


@pytest.mark.slow
def test_select_long_rows_many(lsa):
    """256 queries on rows of 37440 buckets: each row's workgroup walks the spans itself
    (the launch has enough rows); sampled rows bit for bit."""
    prm = (512, 4, 8, 32)
    L = 585 * 512 + 3
    wl = synthetic.Workload("sem_long_many", B=1, n_q=256, L=L, q_pos0=L - 256, H_I=1, d_I=64, k=2048, H_q=16,
                            semantic=True)
    inp = synthetic.semantic_inputs(wl, dev(), seed=14)
    # rows with no scored bucket (inside the first cluster block, or padding) among them
    q_pos = inp["q_pos"].clone()
    q_pos[0, 2], q_pos[0, 3], q_pos[0, 4], q_pos[0, 5] = 100, -1, 0, 511
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    idx, cnt = lsa.lsa_semantic_select(inp["q_sem"], q_pos, cache, 2048, 512, 4, 512)
    torch.cuda.synchronize()
    oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=cache["table"].shape[1])
    for i in (0, 1, 2, 3, 4, 5, 100, 254, 255):
        p = int(q_pos[0, i])
        r = oracle.semantic_select_row(_f32(inp["q_sem"][0, i]), oc, p, 2048, 512, 4, 512)
        assert np.array_equal(idx[0, i].cpu().numpy(), r["J"]), f"i={i}"
        assert int(cnt[0, i]) == r["count"]


@pytest.mark.slow
def test_select_long_rows_past_bitmap(lsa):
    """Rows of few buckets (32 a block, 16416 in all) whose key positions lie past the
    largest position bitmap (513 blocks of 512 keys): the long-row path with spans as
    workgroups of their own, the top-p of 2048 larger than the last span's scores."""
    prm = (512, 4, 16, 64)
    L = 513 * 512 + 9
    wl = synthetic.WORKLOADS["decode_128k_lsa"].replace(B=1, L=L, q_pos0=L - 1)
    positions = [[L - 1]]
    print(f"[long rows past the bitmap {prm} L={L}]", flush=True)
    inp, q, q_pos, cache, idx, cnt = _select_case(lsa, wl, prm, positions, 2048, 2048, 4, 512, seed=15)
    oc = _oracle_cache(inp["k_sem"][0], prm, n_blocks=cache["table"].shape[1])
    r = oracle.semantic_select_row(_f32(q[0, 0]), oc, L - 1, 2048, 2048, 4, 512)
    assert np.array_equal(idx[0, 0].cpu().numpy(), r["J"])
    assert int(cnt[0, 0]) == r["count"]


@pytest.mark.slow
def test_decode_128k_lsa_sampled(lsa):
    """The decode workload at full size (64 sequences, 128K keys each), in the launch
    configuration the benchmark times: sampled cache blocks and two sequences' lists
    bit for bit against the oracle (which clusters those sequences itself)."""
    wl = synthetic.WORKLOADS["decode_128k_lsa"]
    prm = (wl.n_cluster, wl.n_pool, wl.n_bavg, wl.n_bmax)
    inp = synthetic.semantic_inputs(wl, dev())
    print("[decode_128k_lsa] clustering", flush=True)
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm)
    idx, cnt = lsa.lsa_semantic_select(inp["q_sem"], inp["q_pos"], cache, wl.k, wl.p_top, wl.n_sink, wl.n_cluster)
    torch.cuda.synchronize()
    NB = cache["table"].shape[1]
    assert NB == 256
    for b in (0, 37, 63):
        cent, table, offs = _gpu_cache_np(cache, b)
        for t in (0, 1, 128, 255):
            c, tb, of = oracle.sem_cluster_block(_f32(inp["k_sem"][b, t * 512:(t + 1) * 512]), wl.n_pool,
                                                 512 // wl.n_bavg, wl.n_bmax, first_key=t * 512)
            assert np.array_equal(cent[t], c) and np.array_equal(table[t], tb) and np.array_equal(offs[t], of), \
                f"block b={b} t={t}"
    for b in (0, 63):
        print(f"[decode_128k_lsa] oracle cache of sequence {b}", flush=True)
        oc = _oracle_cache(inp["k_sem"][b], prm, n_blocks=NB)
        p = int(inp["q_pos"][b, 0])
        r = oracle.semantic_select_row(_f32(inp["q_sem"][b, 0]), oc, p, wl.k, wl.p_top, wl.n_sink, wl.n_cluster)
        assert np.array_equal(idx[b, 0].cpu().numpy(), r["J"]), f"seq {b}"
        assert int(cnt[b, 0]) == r["count"] == wl.n_sink + wl.k + wl.n_cluster


def test_semantic_decode_graph_replay(lsa):
    """A semantic decode step (selection + attention) captured once in a HIP graph, with
    the cache sized for the longest context, replays for new positions and new index
    queries written into the captured inputs and after a block is clustered into the
    cache between replays; every replay equals an eager call bit for bit."""
    prm = (512, 4, 8, 32)
    k, p_top, n_sink = 256, 64, 4
    L = 24 * 512 + 1
    wl = synthetic.Workload("sgraph", B=4, n_q=1, L=L, q_pos0=L - 1, H_I=1, d_I=64, k=k, H_q=16, semantic=True,
                            p_top=p_top, n_sink=n_sink)
    g = synthetic.make_inputs(wl, dev())
    g.update(synthetic.semantic_inputs(wl, dev(), seed=9))
    g["q_pos"].copy_(torch.tensor([[L - 1], [9000], [600], [5000]], dtype=torch.int32, device=dev()))
    cache = lsa.lsa_semantic_cache(g["k_sem"][:, :20 * 512].contiguous(), *prm, n_blocks=24)
    W = n_sink + k + prm[0]
    idx = torch.empty((4, 1, W), dtype=torch.int32, device=dev())
    cnt = torch.empty((4, 1), dtype=torch.int32, device=dev())
    ws = torch.empty((lsa.lsa_semantic_workspace_size(4, 1, cache),), dtype=torch.uint8, device=dev())

    def step():
        lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache, k, p_top, n_sink, prm[0], idx=idx, count=cnt, ws=ws)
        return lsa.lsa_sparse_attn(g["q"], g["k"], g["v"], idx, scale=wl.scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out, lse = step()
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(11)
    for trial in range(4):
        if trial == 2:   # the next block completes: cluster it into the cache
            lsa.lsa_semantic_cache(g["k_sem"], cache=cache, first_block=20, n_update=4)
        hi = 20 * 512 if trial < 2 else L
        g["q_pos"].copy_(torch.randint(0, hi, (4, 1), generator=gen, dtype=torch.int32).to(dev()))
        g["q_sem"].copy_((g["q_sem"].float() + 0.25 * torch.randn(g["q_sem"].shape, generator=gen).to(dev()))
                         .to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (idx.clone(), cnt.clone(), out.clone(), lse.clone())
        want_idx, want_cnt = lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache, k, p_top, n_sink, prm[0])
        want_out, want_lse = lsa.lsa_sparse_attn(g["q"], g["k"], g["v"], want_idx, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(got[0], want_idx) and torch.equal(got[1], want_cnt), f"replay {trial}: lists"
        assert torch.equal(got[2], want_out) and torch.equal(got[3], want_lse), f"replay {trial}: attention"


def _to_pool(t, pt, P, n_pages, fill_seed):
    """t [B, L, d] scattered over a pool of pages: logical key j of sequence b at row
    pt[b, j // P] * P + j % P; the other rows random."""
    B, L, d = t.shape
    gen = torch.Generator(dev()).manual_seed(fill_seed)
    pool = torch.randn((n_pages * P, d), generator=gen, device=dev()).to(t.dtype)
    j = torch.arange(L, device=dev())
    rows = (pt.long()[:, j // P] * P + j % P).reshape(-1)
    pool.index_copy_(0, rows, t.reshape(B * L, d))
    return pool


def test_semantic_paged(lsa):
    """Paged storage: index keys, K and V in pools of 64-key pages behind a page table, the
    bucket cache in a pool of entries behind a block table.  The cache entries equal the
    contiguous ones slot for slot, the lists are the contiguous lists mapped to pool rows,
    and attention over the pools equals attention over the contiguous caches."""
    prm = (512, 4, 8, 32)
    P, k, p_top = 64, 300, 64
    L = 10 * 512
    wl = synthetic.Workload("sem_paged", B=3, n_q=4, L=L, q_pos0=L - 4, H_I=1, d_I=64, k=k, H_q=16, semantic=True,
                            p_top=p_top, n_sink=4)
    g = synthetic.make_inputs(wl, dev())
    g.update(synthetic.semantic_inputs(wl, dev(), seed=13))
    g["q_pos"].copy_(torch.tensor([[L - 1, 4000, 513, 100], [L - 2, 2047, 3000, 5000], [1024, 1023, 5000, 4777]],
                                  dtype=torch.int32, device=dev()))
    B, NB, max_pages = 3, L // 512, L // P
    gen = torch.Generator().manual_seed(21)
    n_pages = B * max_pages + 17
    pt = torch.randperm(n_pages, generator=gen)[: B * max_pages].view(B, max_pages).to(torch.int32).to(dev())
    n_bslots = B * NB + 5
    bt = torch.randperm(n_bslots, generator=gen)[: B * NB].view(B, NB).to(torch.int32).to(dev())
    k_pool = _to_pool(g["k_sem"], pt, P, n_pages, 1)
    kc_pool, vc_pool = _to_pool(g["k"], pt, P, n_pages, 2), _to_pool(g["v"], pt, P, n_pages, 3)
    paged = {"block_table": bt, "page_table": pt, "page_size": P, "n_slots": n_pages * P}

    cache = lsa.lsa_semantic_cache(g["k_sem"], *prm)
    cache_p = lsa.lsa_semantic_cache(k_pool, *prm, paged=paged, n_bslots=n_bslots)
    idx, cnt = lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache, k, p_top, 4, 512)
    idx_p, cnt_p = lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache_p, k, p_top, 4, 512, paged=paged)
    out, lse = lsa.lsa_sparse_attn(g["q"], g["k"], g["v"], idx, scale=wl.scale)
    out_p, lse_p = lsa.lsa_sparse_attn(g["q"], kc_pool, vc_pool, idx_p, scale=wl.scale)
    torch.cuda.synchronize()
    for name in ("centroids", "table", "offsets"):
        assert torch.equal(cache_p[name][bt.long()], cache[name]), name
    mapped = torch.where(idx >= 0, pt.long().gather(1, (idx.clamp(min=0) // P).view(B, -1)).view_as(idx) * P
                         + idx.clamp(min=0) % P, torch.full_like(idx, -1).long()).to(torch.int32)
    assert torch.equal(idx_p, mapped) and torch.equal(cnt_p, cnt)
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse)
    # the contiguous lists are the oracle's (checked here once more on one sequence)
    oc = _oracle_cache(g["k_sem"][1], prm, n_blocks=NB)
    for i in range(4):
        r = oracle.semantic_select_row(_f32(g["q_sem"][1, i]), oc, int(g["q_pos"][1, i]), k, p_top, 4, 512)
        assert np.array_equal(idx[1, i].cpu().numpy(), r["J"])
        want = np.where(r["J"] >= 0, oracle.paged_rows(pt[1].cpu().numpy(), L, P)[np.maximum(r["J"], 0)], -1)
        assert np.array_equal(idx_p[1, i].cpu().numpy(), want)


def test_semantic_paged_many_rows(lsa):
    """A 600-query chunk over paged storage (the two-workgroups-per-CU selection with
    paging): the contiguous lists mapped to pool rows, bit for bit."""
    prm = (512, 4, 8, 32)
    P = 64
    L = 12 * 512
    wl = synthetic.Workload("sem_paged_chunk", B=1, n_q=600, L=L, q_pos0=L - 600, H_I=1, d_I=64, k=300, H_q=16,
                            semantic=True, p_top=64, n_sink=4)
    g = synthetic.semantic_inputs(wl, dev(), seed=15)
    NB, max_pages = L // 512, L // P
    gen = torch.Generator().manual_seed(23)
    n_pages = max_pages + 9
    pt = torch.randperm(n_pages, generator=gen)[:max_pages].view(1, max_pages).to(torch.int32).to(dev())
    bt = torch.randperm(NB + 3, generator=gen)[:NB].view(1, NB).to(torch.int32).to(dev())
    k_pool = _to_pool(g["k_sem"], pt, P, n_pages, 4)
    paged = {"block_table": bt, "page_table": pt, "page_size": P, "n_slots": n_pages * P}
    cache = lsa.lsa_semantic_cache(g["k_sem"], *prm)
    cache_p = lsa.lsa_semantic_cache(k_pool, *prm, paged=paged, n_bslots=NB + 3)
    idx, cnt = lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache, wl.k, wl.p_top, 4, 512)
    idx_p, cnt_p = lsa.lsa_semantic_select(g["q_sem"], g["q_pos"], cache_p, wl.k, wl.p_top, 4, 512, paged=paged)
    torch.cuda.synchronize()
    mapped = torch.where(idx >= 0, pt.long().gather(1, (idx.clamp(min=0) // P).view(1, -1)).view_as(idx) * P
                         + idx.clamp(min=0) % P, torch.full_like(idx, -1).long()).to(torch.int32)
    assert torch.equal(idx_p, mapped) and torch.equal(cnt_p, cnt)
    with pytest.raises(ValueError):
        lsa.lsa_semantic_cache(k_pool, *prm, paged=paged)
