"""The workloads at full size, in the launch configuration the benchmark times
(lsa_forward with its automatic chunking): sampled rows against the CPU oracle
(indices bit-exact, attention within tolerance) and, on every row the GPU memory
allows, the O(n) top-k certificate over the GPU's own scores."""
from __future__ import annotations

import math
import time

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import AttnErr, dev, np64, topk_certificate

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def lsa():
    import learned_top_sparse_amd as m
    m.lib()
    return m


def _run(lsa, name):
    wl = synthetic.WORKLOADS[name]
    g = synthetic.make_inputs(wl, dev())
    t0 = time.time()
    res = lsa.lsa_forward(g, k_top=wl.k, two_stage=wl.two_stage, block_size=wl.block_size, n_keep=wl.n_keep)
    torch.cuda.synchronize()
    print(f"[{name}] forward {time.time() - t0:.3f}s", flush=True)
    return wl, g, res


def _check_rows(wl, g, res, rows):
    qi = g["q_idx"]
    err = AttnErr()
    J = res["idx"]
    out = res["out"]
    w = g["w"].cpu().numpy()
    batches = sorted({b for b, _ in rows})
    t0 = time.time()
    for b in batches:
        ki = g["k_idx"][b].cpu().numpy()
        kk = g["k"][b].cpu()
        vv = g["v"][b].cpu()
        reps = oracle.block_reps(ki, wl.block_size) if wl.two_stage else None
        for (bb, i) in [r for r in rows if r[0] == b]:
            p = int(g["q_pos"][b, i])
            r = oracle.forward_row(qi[b, i].cpu().numpy(), ki, w, p, wl.k, two_stage=wl.two_stage,
                                   block_size=wl.block_size, n_keep=wl.n_keep, reps=reps)
            Jg = J[b, i].cpu().numpy()
            assert np.array_equal(Jg, r["J"]), f"{wl.name}: index list of row {(b, i)} (p={p}) differs"
            if wl.two_stage:
                assert np.array_equal(res["kept"][b, i].cpu().numpy(), r["kept"]), f"kept row {(b, i)}"
            # attention over the (identical) list, fp64 on the bf16-cast inputs
            Jv = r["J"][r["J"] >= 0]
            o, _ = oracle.sparse_attention(np64(g["q"][b, i]), np64(kk[Jv]), np64(vv[Jv]), np.arange(Jv.size),
                                           wl.scale)
            err.add(np64(out[b, i]), o, (b, i))
    print(f"[{wl.name}] oracle checked {len(rows)} rows in {time.time() - t0:.1f}s; "
          f"attn max-abs {err.max_abs:.2e} rel-L2 {err.rel_l2:.2e}", flush=True)
    err.check()


def _certificate_flat(lsa, wl, g, res, row_chunk):
    """Recompute the GPU scores chunk by chunk and certify every listed row."""
    B, n_q = wl.B, wl.n_q
    for b in range(B):
        for i0 in range(0, n_q, row_chunk):
            i1 = min(n_q, i0 + row_chunk)
            sl = lambda t: t[b: b + 1, i0:i1].contiguous()
            S = lsa.lsa_index_scores(sl(g["q_idx"]), g["k_idx"][b: b + 1].contiguous(), g["w"], sl(g["q_pos"]))
            topk_certificate(S[0], res["idx"][b, i0:i1], g["q_pos"][b, i0:i1], wl.k)


def test_prefill_32k(lsa):
    wl, g, res = _run(lsa, "prefill_32k")
    _check_rows(wl, g, res, synthetic.checked_rows(wl))
    _certificate_flat(lsa, wl, g, res, row_chunk=2048)


def _pool_rows(J, page_table, P):
    """Logical keys [B, n_q, k] (or -1) -> pool rows through page_table [B, max_pages]."""
    J = J.long()
    Jc = J.clamp(min=0)
    rows = torch.gather(page_table.long(), 1, (Jc // P).reshape(J.shape[0], -1)).reshape(J.shape) * P + Jc % P
    return torch.where(J >= 0, rows, torch.full_like(J, -1))


def _paged_equal(lsa, name, g, res, **kw):
    """The benchmark's paged variant of a workload (its caches scattered over a pool of
    pages) gives the contiguous step bit for bit, the lists naming pool rows."""
    wp = synthetic.WORKLOADS[name]
    pg = synthetic.paged_pool(g, wp.page_size, wp.spare_pages, wp.seed)
    if wp.pooled:
        pg["block_keys"] = lsa.lsa_block_cache(pg["k_idx"], wp.block_size, page_table=pg["page_table"],
                                               page_size=wp.page_size)
    rp = lsa.lsa_forward(pg, k_top=wp.k, **kw)
    torch.cuda.synchronize()
    assert torch.equal(rp["idx"].long(), _pool_rows(res["idx"], pg["page_table"], wp.page_size))
    for n in ("count", "out", "lse", "kept"):
        if n in res:
            assert torch.equal(rp[n], res[n]), n
    print(f"[{name}] equal to the contiguous step", flush=True)


def test_decode_128k(lsa):
    wl, g, res = _run(lsa, "decode_128k")
    _check_rows(wl, g, res, synthetic.checked_rows(wl, n_random=10))
    S = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"])
    topk_certificate(S[:, 0], res["idx"][:, 0], g["q_pos"][:, 0], wl.k)
    del S
    # the benchmark's paged variant (decode_128k_paged): the same caches scattered over a
    # pool of 64-token pages give the same step, the lists naming pool rows
    wp = synthetic.WORKLOADS["decode_128k_paged"]
    pg = synthetic.paged_pool(g, wp.page_size, wp.spare_pages, wp.seed)
    rp = lsa.lsa_forward(pg, k_top=wp.k)
    torch.cuda.synchronize()
    P = wp.page_size
    J = res["idx"].long()
    pt = pg["page_table"].long()
    Jc = J.clamp(min=0)
    rows = torch.gather(pt, 1, (Jc // P).reshape(wl.B, -1)).reshape(J.shape) * P + Jc % P
    assert torch.equal(rp["idx"].long(), torch.where(J >= 0, rows, torch.full_like(J, -1)))
    assert torch.equal(rp["out"], res["out"]) and torch.equal(rp["lse"], res["lse"])
    print("[decode_128k_paged] equal to the contiguous step", flush=True)


def test_chunk_256k(lsa):
    wl, g, res = _run(lsa, "chunk_256k")
    _check_rows(wl, g, res, synthetic.checked_rows(wl))
    # certificate on a seeded 1024-row subset (scores of all 16384 rows would be 17 GB)
    rng = np.random.default_rng(1)
    for i0 in sorted(rng.choice(wl.n_q // 256, size=4, replace=False) * 256):
        sl = lambda t: t[:, i0: i0 + 256].contiguous()
        S = lsa.lsa_index_scores(sl(g["q_idx"]), g["k_idx"], g["w"], sl(g["q_pos"]))
        topk_certificate(S[0], res["idx"][0, i0: i0 + 256], g["q_pos"][0, i0: i0 + 256], wl.k)


def test_two_stage_128k(lsa):
    wl, g, res = _run(lsa, "two_stage_128k")
    _check_rows(wl, g, res, synthetic.checked_rows(wl))
    # certificate of every row's token top-k inside its kept blocks
    bs, nk = wl.block_size, wl.n_keep
    kept = res["kept"]
    S = lsa.lsa_index_scores(g["q_idx"], g["k_idx"], g["w"], g["q_pos"], kept_blocks=kept, block_size=bs)
    slots = torch.arange(nk * bs, device=S.device)
    blk = kept[0][:, slots // bs].to(torch.int64)
    keys = blk * bs + (slots % bs)
    valid = (blk >= 0) & (keys <= g["q_pos"][0].to(torch.int64).unsqueeze(1))
    topk_certificate(S[0], res["idx"][0], g["q_pos"][0], wl.k, keys=keys, valid=valid)
    # certificate of the block keep itself: own kept, ascending, and kept blocks beat the rest
    reps = lsa.lsa_block_reps(g["k_idx"], bs)
    _, bsc = lsa.lsa_block_prefilter(g["q_idx"], reps, g["w"], g["q_pos"], bs, nk, return_scores=True)
    own = (g["q_pos"][0] // bs).to(torch.int64)
    kp = kept[0].to(torch.int64)
    assert bool((kp.max(1).values == own).all())
    n_blocks = bsc.shape[-1]
    m = torch.arange(n_blocks, device=S.device).unsqueeze(0)
    earlier = m < own.unsqueeze(1)
    hits = torch.zeros(earlier.shape, dtype=torch.int32, device=S.device)
    hits.scatter_add_(1, torch.clamp(kp, min=0), (kp >= 0).to(torch.int32))
    is_kept = hits > 0
    packed_lo = bsc[0].clone()
    big = torch.iinfo(torch.int64).max
    # kept blocks score at least as high as the dropped ones (exact ties are settled by the
    # sampled rows above, which compare the lists with the oracle element by element)
    sel = earlier & is_kept
    oth = earlier & ~is_kept
    min_sel = torch.where(sel, packed_lo, torch.full_like(packed_lo, big)).min(1).values
    max_oth = torch.where(oth, packed_lo, torch.full_like(packed_lo, -big - 1)).max(1).values
    assert bool(((min_sel >= max_oth) | (oth.sum(1) == 0)).all())
    assert bool((sel.sum(1) == torch.clamp(own, max=nk - 1)).all())
    del S, bsc, hits
    _paged_equal(lsa, "two_stage_128k_paged", g, res, two_stage=True, block_size=bs, n_keep=nk)


@pytest.mark.parametrize("name", ["prefill_32k_pool4", "chunk_256k_pool4"])
def test_prefill_pool4(lsa, name):
    """The pooled (4:1) indexer on the prefill workloads at full size, with the block-key
    cache built beforehand as the benchmark does: seeded sampled rows (boundary rows
    included) against the oracle -- lists, kept blocks and counts exact, attention within
    tolerance."""
    wl = synthetic.WORKLOADS[name]
    g = synthetic.make_inputs(wl, dev())
    g["block_keys"] = lsa.lsa_block_cache(g["k_idx"], wl.block_size)
    t0 = time.time()
    res = lsa.lsa_forward(g, k_top=wl.k, two_stage="pooled", block_size=wl.block_size, n_keep=wl.n_keep)
    torch.cuda.synchronize()
    print(f"[{wl.name}] forward {time.time() - t0:.3f}s", flush=True)
    w = g["w"].cpu().numpy()
    ki = g["k_idx"][0].cpu().numpy()
    kc, vc = np64(g["k"][0].cpu()), np64(g["v"][0].cpu())
    reps = oracle.block_reps(ki, wl.block_size)
    err = AttnErr()
    for b, i in synthetic.checked_rows(wl, n_random=12):
        p = int(g["q_pos"][b, i])
        r = oracle.forward_row(g["q_idx"][b, i].cpu().numpy(), ki, w, p, wl.k, q_row=np64(g["q"][b, i]),
                               k_cache=kc, v_cache=vc, scale=wl.scale, two_stage=True, block_size=wl.block_size,
                               n_keep=wl.n_keep, pooled=True, reps=reps)
        assert np.array_equal(res["kept"][b, i].cpu().numpy(), r["kept"]), f"kept {(b, i)}"
        assert np.array_equal(res["idx"][b, i].cpu().numpy(), r["J"]), f"row {(b, i)}"
        assert int(res["count"][b, i]) == r["count"]
        err.add(np64(res["out"][b, i]), r["out"], (b, i))
    err.check()


def test_decode_128k_pool4(lsa):
    """The pooled (4:1) decode workload at full size, with the block-key cache built
    beforehand as the benchmark does: sampled rows against the oracle (lists, kept
    blocks and counts exact, attention within tolerance)."""
    wl = synthetic.WORKLOADS["decode_128k_pool4"]
    g = synthetic.make_inputs(wl, dev())
    g["block_keys"] = lsa.lsa_block_cache(g["k_idx"], wl.block_size)
    t0 = time.time()
    res = lsa.lsa_forward(g, k_top=wl.k, two_stage="pooled", block_size=wl.block_size, n_keep=wl.n_keep)
    torch.cuda.synchronize()
    print(f"[{wl.name}] forward {time.time() - t0:.3f}s", flush=True)
    w = g["w"].cpu().numpy()
    err = AttnErr()
    for b, _ in synthetic.checked_rows(wl, n_random=6):
        ki = g["k_idx"][b].cpu().numpy()
        p = int(g["q_pos"][b, 0])
        r = oracle.forward_row(g["q_idx"][b, 0].cpu().numpy(), ki, w, p, wl.k, q_row=np64(g["q"][b, 0]),
                               k_cache=np64(g["k"][b].cpu()), v_cache=np64(g["v"][b].cpu()), scale=wl.scale,
                               two_stage=True, block_size=wl.block_size, n_keep=wl.n_keep, pooled=True)
        assert np.array_equal(res["idx"][b, 0].cpu().numpy(), r["J"]), f"seq {b}"
        assert np.array_equal(res["kept"][b, 0].cpu().numpy(), r["kept"]), f"kept {b}"
        assert int(res["count"][b, 0]) == r["count"]
        err.add(np64(res["out"][b, 0]), r["out"], b)
    err.check()
    del g["block_keys"]
    _paged_equal(lsa, "decode_128k_pool4_paged", g, res, two_stage="pooled", block_size=wl.block_size,
                 n_keep=wl.n_keep)
