"""Seeded synthetic inputs for the indexer -> exact top-k -> sparse-attention path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds shapes and random draws only: none of the method's
arithmetic lives here, so neither side can borrow the other's through it.

Value distributions (the workloads described for the path):
  * index queries / keys: int8, uniform over the integers -64..64 inclusive;
  * indexer head weights w_h: int32, uniform over 1..16 inclusive;
  * attention Q, K, V: fp32 draws from N(0, 1), cast to bf16 with
    round-to-nearest-even.

Each tensor has its own torch.Generator seeded with ``seed * 16 + id``
(q_idx=1, k_idx=2, w=3, q=4, k=5, v=6), so a tensor does not depend on which
others were drawn.  Draws are made on the device the caller names; CPU and GPU
streams differ, so a test always hands the oracle a host copy of exactly the
tensors the GPU consumed.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

IDS = {"q_idx": 1, "k_idx": 2, "w": 3, "q": 4, "k": 5, "v": 6,
       "pages": 7, "pool_k_idx": 8, "pool_k": 9, "pool_v": 10,
       "sem_topics": 11, "k_sem": 12, "q_sem": 13, "sem_blocks": 14, "pool_k_sem": 15}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one workload of the path.

    ``q_pos0`` is the absolute position of the first query of the chunk; query
    i of every sequence sits at ``q_pos0 + i`` and sees keys 0..q_pos0+i.
    ``L`` is the number of cached tokens (keys) per sequence.
    """
    name: str
    B: int
    n_q: int
    L: int
    q_pos0: int
    H_I: int
    d_I: int
    k: int
    H_q: int
    d: int = 128
    two_stage: bool = False
    block_size: int = 128
    n_keep: int = 64
    seed: int = 0
    pooled: bool = False    # two_stage with the kept blocks' keys as the list (k = n_keep * block_size)
    page_size: int = 0      # > 0: caches scattered over a pool of pages (paged_pool)
    spare_pages: int = 0    # unused pool pages besides the sequences' own
    semantic: bool = False  # flat semantic search: bf16 index keys / queries of 64 dims
    n_cluster: int = 512    # keys per cluster block (the window is one block)
    n_pool: int = 4         # keys per pool key
    n_bavg: int = 8         # average keys per bucket
    n_bmax: int = 32        # largest bucket (keys)
    p_top: int = 512        # buckets kept per query (p * n_pool >= k)
    n_sink: int = 4         # sink keys

    @property
    def decode(self) -> bool:
        return self.n_q == 1 and self.B > 1

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of the path.  Names say what each one is.
WORKLOADS = {
    # tiny causal prefill: small enough for the oracle to check every row
    "tiny_prefill_1k": Workload("tiny_prefill_1k", B=1, n_q=1024, L=1024, q_pos0=0,
                                H_I=4, d_I=64, k=64, H_q=8),
    # causal prefill of a 32K-token context
    "prefill_32k": Workload("prefill_32k", B=1, n_q=32768, L=32768, q_pos0=0,
                            H_I=64, d_I=128, k=2048, H_q=16),
    # decode: 64 sequences, 131072 cached tokens + the new one each
    "decode_128k": Workload("decode_128k", B=64, n_q=1, L=131073, q_pos0=131072,
                            H_I=64, d_I=128, k=2048, H_q=16),
    # last 16384-query chunk of a 262144-token context (one GPU's share)
    "chunk_256k": Workload("chunk_256k", B=1, n_q=16384, L=262144, q_pos0=245760,
                           H_I=64, d_I=128, k=2048, H_q=16),
    # decode_128k with its caches scattered over a pool of 64-token pages (serving layout)
    "decode_128k_paged": Workload("decode_128k_paged", B=64, n_q=1, L=131073, q_pos0=131072,
                                  H_I=64, d_I=128, k=2048, H_q=16, page_size=64, spare_pages=4096),
    # decode_128k with a 4:1 pooled indexer: one pooled key per 4 keys, the best 512 blocks
    # (own block included) give the 2048-key list
    "decode_128k_pool4": Workload("decode_128k_pool4", B=64, n_q=1, L=131073, q_pos0=131072,
                                  H_I=64, d_I=128, k=2048, H_q=16, two_stage=True, pooled=True,
                                  block_size=4, n_keep=512),
    # decode_128k_pool4 over the page pool of decode_128k_paged
    "decode_128k_pool4_paged": Workload("decode_128k_pool4_paged", B=64, n_q=1, L=131073, q_pos0=131072,
                                        H_I=64, d_I=128, k=2048, H_q=16, two_stage=True, pooled=True,
                                        block_size=4, n_keep=512, page_size=64, spare_pages=4096),
    # the 32K prefill and the 256K chunk with the 4:1 pooled indexer (the best 512 blocks
    # of 4 keys, own block included, give the 2048-key list)
    "prefill_32k_pool4": Workload("prefill_32k_pool4", B=1, n_q=32768, L=32768, q_pos0=0,
                                  H_I=64, d_I=128, k=2048, H_q=16, two_stage=True, pooled=True,
                                  block_size=4, n_keep=512),
    "chunk_256k_pool4": Workload("chunk_256k_pool4", B=1, n_q=16384, L=262144, q_pos0=245760,
                                 H_I=64, d_I=128, k=2048, H_q=16, two_stage=True, pooled=True,
                                 block_size=4, n_keep=512),
    # two-stage (block prefilter, then tokens) on the final 8192 queries of 128K
    "two_stage_128k": Workload("two_stage_128k", B=1, n_q=8192, L=131072, q_pos0=122880,
                               H_I=64, d_I=128, k=2048, H_q=16, two_stage=True,
                               block_size=128, n_keep=64),
    # two_stage_128k with its caches in a pool of 64-token pages (1024 spare pages)
    "two_stage_128k_paged": Workload("two_stage_128k_paged", B=1, n_q=8192, L=131072, q_pos0=122880,
                                     H_I=64, d_I=128, k=2048, H_q=16, two_stage=True,
                                     block_size=128, n_keep=64, page_size=64, spare_pages=1024),
    # flat semantic search (bucket cache of 512-key blocks, 64 buckets each): decode of 64
    # sequences at 128K, 2048 long-range keys from the best 512 buckets + 4 sinks + a
    # 512-key window
    "decode_128k_lsa": Workload("decode_128k_lsa", B=64, n_q=1, L=131073, q_pos0=131072,
                                H_I=1, d_I=64, k=2048, H_q=16, semantic=True),
    # decode_128k_lsa over paged storage: keys, K and V in pools of 64-token pages (4096
    # spare pages), the bucket cache in a pool of entries behind a block table
    "decode_128k_lsa_paged": Workload("decode_128k_lsa_paged", B=64, n_q=1, L=131073, q_pos0=131072,
                                      H_I=1, d_I=64, k=2048, H_q=16, semantic=True, page_size=64,
                                      spare_pages=4096),
    # semantic decode at 1M context: 8 sequences of 1048576 cached keys (131072 buckets a row)
    "decode_1m_lsa": Workload("decode_1m_lsa", B=8, n_q=1, L=1048577, q_pos0=1048576,
                              H_I=1, d_I=64, k=2048, H_q=16, semantic=True),
    # the same search for the final 8192 queries of a 128K prefill
    "prefill_128k_lsa": Workload("prefill_128k_lsa", B=1, n_q=8192, L=131072, q_pos0=122880,
                                 H_I=1, d_I=64, k=2048, H_q=16, semantic=True),
}


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + tid)
    return g


def _randint(shape, lo, hi_incl, dtype, seed, tid, device, chunk_rows=1 << 26):
    """Uniform integers in [lo, hi_incl], drawn row-chunk by row-chunk."""
    g = _gen(seed, tid, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    step = chunk_rows
    for s in range(0, n, step):
        e = min(n, s + step)
        flat[s:e] = torch.randint(lo, hi_incl + 1, (e - s,), generator=g,
                                  device=device, dtype=torch.int32).to(dtype)
    return out


def _randn_bf16(shape, seed, tid, device, chunk=1 << 26):
    g = _gen(seed, tid, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn((e - s,), generator=g, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def q_positions(wl: Workload, device="cpu") -> torch.Tensor:
    """int32 [B, n_q]: absolute position of every query."""
    pos = torch.arange(wl.n_q, dtype=torch.int32, device=device) + wl.q_pos0
    return pos.unsqueeze(0).expand(wl.B, wl.n_q).contiguous()


def make_inputs(wl: Workload, device="cpu", with_attn: bool = True,
                seed: Optional[int] = None) -> dict:
    """Draw every input of ``wl`` on ``device``.

    Returns a dict of contiguous tensors:
      q_idx int8 [B, n_q, H_I, d_I], k_idx int8 [B, L, d_I], w int32 [H_I],
      q_pos int32 [B, n_q] and, if ``with_attn``, q bf16 [B, n_q, H_q, d],
      k / v bf16 [B, L, d].
    """
    s = wl.seed if seed is None else seed
    out = {
        "q_idx": _randint((wl.B, wl.n_q, wl.H_I, wl.d_I), -64, 64, torch.int8, s, IDS["q_idx"], device),
        "k_idx": _randint((wl.B, wl.L, wl.d_I), -64, 64, torch.int8, s, IDS["k_idx"], device),
        "w": _randint((wl.H_I,), 1, 16, torch.int32, s, IDS["w"], device),
        "q_pos": q_positions(wl, device),
    }
    if with_attn:
        out["q"] = _randn_bf16((wl.B, wl.n_q, wl.H_q, wl.d), s, IDS["q"], device)
        out["k"] = _randn_bf16((wl.B, wl.L, wl.d), s, IDS["k"], device)
        out["v"] = _randn_bf16((wl.B, wl.L, wl.d), s, IDS["v"], device)
    if wl.page_size > 0:
        return paged_pool(out, wl.page_size, wl.spare_pages, s)
    return out


def paged_pool(inp: dict, page_size: int, spare_pages: int = 0, seed: int = 0) -> dict:
    """The caches of ``inp`` scattered over one shared pool of pages (serving layout).

    Sequence b's L keys fill max_pages = ceil(L / page_size) pages.  Those B * max_pages
    pages and ``spare_pages`` unused ones are laid out in a seeded random order, so
    sequence b's page m sits at pool page page_table[b, m].  Returns a copy of ``inp``
    whose k_idx, k and v are pools [n_slots, .] (n_slots = pages * page_size) holding
    the keys of ``inp`` at the rows the page table names and seeded random values
    elsewhere (spare pages, the tail of each last page), plus page_table (int32
    [B, max_pages]) and page_size.  It moves data only.
    """
    k_idx = inp["k_idx"]
    device = k_idx.device
    B, L, d_I = k_idx.shape
    max_pages = -(-L // page_size)
    n_pages = B * max_pages + spare_pages
    g = torch.Generator().manual_seed(seed * 16 + IDS["pages"])
    order = torch.randperm(n_pages, generator=g)[: B * max_pages].to(torch.int32)
    page_table = order.view(B, max_pages).contiguous().to(device)
    n_slots = n_pages * page_size
    j = torch.arange(L, device=device, dtype=torch.int64)
    rows = (page_table.long()[:, j // page_size] * page_size + j % page_size).reshape(-1)
    out = dict(inp)
    out["k_idx"] = _randint((n_slots, d_I), -64, 64, torch.int8, seed, IDS["pool_k_idx"], device)
    out["k_idx"].index_copy_(0, rows, k_idx.reshape(B * L, d_I))
    for name in ("k", "v"):
        if name in inp:
            t = inp[name]
            pool = _randn_bf16((n_slots, t.shape[-1]), seed, IDS["pool_" + name], device)
            pool.index_copy_(0, rows, t.reshape(B * L, t.shape[-1]))
            out[name] = pool
    out["page_table"] = page_table
    out["page_size"] = page_size
    return out


def semantic_inputs(wl: Workload, device="cpu", seed: Optional[int] = None, n_topics: int = 64,
                    noise: float = 0.5) -> dict:
    """Index keys and queries of flat semantic search (bf16, 64 dims) with topic structure:
    a sequence is a run of spans of 16..127 tokens, each on one of ``n_topics`` topics;
    a key is its topic's centre (N(0, 1) per dim) plus N(0, noise^2) noise, a query the
    centre of a random topic plus the same noise.  Returns dict(k_sem [B, L, 64],
    q_sem [B, n_q, 64], q_pos)."""
    s = wl.seed if seed is None else seed
    gt = _gen(s, IDS["sem_topics"], "cpu")
    centres = torch.randn((n_topics, 64), generator=gt)
    topic = torch.empty((wl.B, wl.L), dtype=torch.int64)
    for b in range(wl.B):
        lens = torch.randint(16, 128, (wl.L // 16 + 1,), generator=gt)
        tops = torch.randint(0, n_topics, (lens.shape[0],), generator=gt)
        topic[b] = torch.repeat_interleave(tops, lens)[: wl.L]
    q_topic = torch.randint(0, n_topics, (wl.B, wl.n_q), generator=gt)
    gk = _gen(s, IDS["k_sem"], device)
    gq = _gen(s, IDS["q_sem"], device)
    c = centres.to(device)
    k_sem = torch.empty((wl.B, wl.L, 64), dtype=torch.bfloat16, device=device)
    for b in range(wl.B):
        k_sem[b] = (c[topic[b].to(device)] + noise * torch.randn((wl.L, 64), generator=gk, device=device,
                                                                 dtype=torch.float32)).to(torch.bfloat16)
    q_sem = (c[q_topic.to(device)] + noise * torch.randn((wl.B, wl.n_q, 64), generator=gq, device=device,
                                                         dtype=torch.float32)).to(torch.bfloat16)
    return {"k_sem": k_sem, "q_sem": q_sem, "q_pos": q_positions(wl, device)}


def semantic_paged(inp: dict, page_size: int, spare_pages: int, n_blocks: int, seed: int = 0) -> dict:
    """The semantic inputs of ``inp`` (k_sem, k, v: [B, L, .]) over paged storage: the
    caches scattered over pools of pages in a seeded order (as paged_pool), and a block
    table naming, in a seeded order, the bucket-cache entry of each of the n_blocks
    cluster blocks of every sequence (a pool of B * n_blocks + 16 entries).  Returns a
    copy with k_sem, k, v replaced by pools [n_slots, .] and paged = dict(block_table,
    page_table, page_size, n_slots), n_bslots.  It moves data only."""
    k_sem = inp["k_sem"]
    device = k_sem.device
    B, L, _ = k_sem.shape
    max_pages = -(-L // page_size)
    n_pages = B * max_pages + spare_pages
    g = torch.Generator().manual_seed(seed * 16 + IDS["pages"])
    page_table = torch.randperm(n_pages, generator=g)[: B * max_pages].to(torch.int32).view(B, max_pages)
    page_table = page_table.contiguous().to(device)
    n_slots = n_pages * page_size
    j = torch.arange(L, device=device, dtype=torch.int64)
    rows = (page_table.long()[:, j // page_size] * page_size + j % page_size).reshape(-1)
    out = dict(inp)
    for name, tid in (("k_sem", "pool_k_sem"), ("k", "pool_k"), ("v", "pool_v")):
        t = inp[name]
        pool = _randn_bf16((n_slots, t.shape[-1]), seed, IDS[tid], device)
        pool.index_copy_(0, rows, t.reshape(B * L, t.shape[-1]))
        out[name] = pool
    gb = torch.Generator().manual_seed(seed * 16 + IDS["sem_blocks"])
    n_bslots = B * n_blocks + 16
    block_table = torch.randperm(n_bslots, generator=gb)[: B * n_blocks].to(torch.int32).view(B, n_blocks)
    out["paged"] = {"block_table": block_table.contiguous().to(device), "page_table": page_table,
                    "page_size": page_size, "n_slots": n_slots}
    out["n_bslots"] = n_bslots
    return out


def checked_rows(wl: Workload, n_random: int = 56, seed: int = 0) -> list:
    """Seeded subset of (b, i) query rows for the large workloads.

    Always includes the first and last row of the chunk; for prefills starting
    at position 0 also the rows at positions k-2, k-1, k (where the candidate
    count crosses the budget); for two-stage workloads rows at the first and
    last position of a key block.
    """
    rng = torch.Generator().manual_seed(seed * 16 + 15)
    rows = set()
    if wl.n_q == 1:
        # decode: whole sequences; 0 and B-1 plus seeded others
        picks = torch.randperm(wl.B, generator=rng)[: max(0, min(n_random, wl.B) - 2)].tolist()
        for b in [0, wl.B - 1] + picks:
            rows.add((b, 0))
        return sorted(rows)
    for i in [0, wl.n_q - 1]:
        rows.add((0, i))
    if wl.q_pos0 == 0:
        for p in (wl.k - 2, wl.k - 1, wl.k):
            if 0 <= p < wl.n_q:
                rows.add((0, p))
    if wl.two_stage:
        bs = wl.block_size
        for p in (wl.q_pos0 + 5 * bs, wl.q_pos0 + 5 * bs + bs - 1):
            i = p - wl.q_pos0
            if 0 <= i < wl.n_q:
                rows.add((0, i))
    b_idx = torch.randint(0, wl.B, (n_random,), generator=rng).tolist()
    i_idx = torch.randint(0, wl.n_q, (n_random,), generator=rng).tolist()
    for b, i in zip(b_idx, i_idx):
        rows.add((b, i))
    return sorted(rows)
