"""ctypes binding of liblsa.so with the C ABI's names (see include/lsa.h).

Argument marshalling only: dtype / device / contiguity checks, output and
workspace allocation through torch, raw device pointers, the current stream.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from typing import Optional

import torch

from .abi import EXPORTED, I32, I64, NOALLOC_SCRATCH_BYTES, P, SZ, ForwardArgs, SemanticPages, SemanticParams, declare

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

STAGE_NAMES = {1: "block_reps", 2: "block_prefilter", 3: "index_select", 4: "index_scores", 5: "topk", 7: "sample",
               6: "sparse_attn", 8: "expand"}


class LsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({lsa_status_string(status)})")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, "liblsa.so")


def lib():
    """The loaded liblsa.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = C.CDLL(path)
        declare(L)
        _LIB = L
    return _LIB


def lsa_status_string(status: int) -> str:
    return lib().lsa_status_string(int(status)).decode()


def lsa_version() -> int:
    return int(lib().lsa_version())


def _check(fn: str, status: int):
    if status != 0:
        raise LsaError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- calls
def lsa_index_scores(q_idx, k_idx, w, q_pos, scores=None, ld: Optional[int] = None,
                     kept_blocks=None, block_size: int = 0, n_keep: int = 0):
    """Indexer scores.  Flat: int32 [B, n_q, ld >= L]; two-stage (kept_blocks):
    compact slots [B, n_q, ld >= n_keep*block_size].  Returns the score tensor."""
    dev = q_idx.device
    _need(q_idx, "q_idx", torch.int8)
    _need(k_idx, "k_idx", torch.int8, dev)
    _need(w, "w", torch.int32, dev)
    _need(q_pos, "q_pos", torch.int32, dev)
    B, n_q, H_I, d_I = q_idx.shape
    L = k_idx.shape[1]
    if k_idx.shape != (B, L, d_I):
        raise ValueError("k_idx must be [B, L, d_I]")
    w_pq = 1 if w.dim() == 3 else 0
    if (w_pq and tuple(w.shape) != (B, n_q, H_I)) or (not w_pq and tuple(w.shape) != (H_I,)):
        raise ValueError("w must be [H_I] or [B, n_q, H_I]")
    if kept_blocks is not None:
        _need(kept_blocks, "kept_blocks", torch.int32, dev)
        n_keep = kept_blocks.shape[-1]
        width = n_keep * block_size
    else:
        width = L
    if ld is None:
        ld = width
    if scores is None:
        scores = torch.empty((B, n_q, ld), dtype=torch.int32, device=dev)
    _need(scores, "scores", torch.int32, dev)
    st = lib().lsa_index_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w), w_pq, _ptr(q_pos), _ptr(kept_blocks),
                                block_size, n_keep, B, n_q, L, H_I, d_I, _ptr(scores), ld, _stream(dev))
    _check("lsa_index_scores", st)
    return scores


def lsa_block_reps(k_idx, block_size: int, n_blocks: Optional[int] = None):
    dev = k_idx.device
    _need(k_idx, "k_idx", torch.int8)
    B, L, d_I = k_idx.shape
    if n_blocks is None:
        n_blocks = L // block_size
    reps = torch.empty((B, n_blocks, d_I), dtype=torch.int32, device=dev)
    st = lib().lsa_block_reps(_ptr(k_idx), B, L, d_I, block_size, n_blocks, _ptr(reps), _stream(dev))
    _check("lsa_block_reps", st)
    return reps


def lsa_block_cache(k_idx, block_size: int, n_blocks: Optional[int] = None, out: Optional[torch.Tensor] = None,
                    first_block: int = 0, n_update: Optional[int] = None, page_table=None, page_size: int = 0):
    """Block-key cache int8 [B, n_blocks, 2, d_I] (hi, lo parts of each block's key sum);
    with ``out`` given, only blocks [first_block, first_block + n_update) are (re)written.
    With ``page_table`` (int32 [B, max_pages]) and ``page_size``, k_idx is a pool
    [n_slots, d_I] read through the page table (lsa_block_cache_paged)."""
    dev = k_idx.device
    _need(k_idx, "k_idx", torch.int8)
    if page_table is not None:
        _need(page_table, "page_table", torch.int32, dev)
        B, max_pages = page_table.shape
        L, d_I = max_pages * page_size, k_idx.shape[1]
    else:
        B, L, d_I = k_idx.shape
    if n_blocks is None:
        n_blocks = L // block_size
    if out is None:
        out = torch.empty((B, n_blocks, 2, d_I), dtype=torch.int8, device=dev)
    _need(out, "block_keys", torch.int8, dev)
    if n_update is None:
        n_update = n_blocks - first_block
    if page_table is not None:
        st = lib().lsa_block_cache_paged(_ptr(k_idx), k_idx.shape[0], _ptr(page_table), page_size, max_pages, B,
                                         d_I, block_size, n_blocks, first_block, n_update, _ptr(out), _stream(dev))
        _check("lsa_block_cache_paged", st)
        return out
    st = lib().lsa_block_cache(_ptr(k_idx), B, L, d_I, block_size, n_blocks, first_block, n_update, _ptr(out),
                               _stream(dev))
    _check("lsa_block_cache", st)
    return out


def lsa_block_prefilter(q_idx, reps, w, q_pos, block_size: int, n_keep: int, return_scores: bool = False):
    """Kept blocks int32 [B, n_q, n_keep] (ascending, -1 padded); optionally block scores int64."""
    dev = q_idx.device
    _need(q_idx, "q_idx", torch.int8)
    _need(reps, "reps", torch.int32, dev)
    _need(w, "w", torch.int32, dev)
    _need(q_pos, "q_pos", torch.int32, dev)
    B, n_q, H_I, d_I = q_idx.shape
    n_blocks = reps.shape[1]
    w_pq = 1 if w.dim() == 3 else 0
    kept = torch.empty((B, n_q, n_keep), dtype=torch.int32, device=dev)
    bs = torch.empty((B, n_q, n_blocks), dtype=torch.int64, device=dev) if return_scores else None
    nb = SZ(0)
    _check("lsa_block_prefilter_workspace_size",
           lib().lsa_block_prefilter_workspace_size(B, n_q, n_blocks, d_I, C.byref(nb)))
    ws = _workspace(nb.value, dev)
    st = lib().lsa_block_prefilter(_ptr(q_idx), _ptr(reps), _ptr(w), w_pq, _ptr(q_pos), B, n_q, n_blocks, H_I,
                                   d_I, block_size, n_keep, _ptr(kept), _ptr(bs), _ptr(ws), nb.value,
                                   _stream(dev))
    _check("lsa_block_prefilter", st)
    return (kept, bs) if return_scores else kept


def lsa_topk(scores, q_pos, k: int, L_max: int, kept_blocks=None, block_size: int = 0, use_ws: bool = True):
    """Exact top-k: (idx int32 [B, n_q, k] ascending and -1 padded, count int32 [B, n_q])."""
    dev = scores.device
    _need(scores, "scores", torch.int32)
    _need(q_pos, "q_pos", torch.int32, dev)
    B, n_q, ld = scores.shape
    n_keep = 0
    if kept_blocks is not None:
        _need(kept_blocks, "kept_blocks", torch.int32, dev)
        n_keep = kept_blocks.shape[-1]
    idx = torch.empty((B, n_q, k), dtype=torch.int32, device=dev)
    count = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    nb = SZ(0)
    _check("lsa_topk_workspace_size", lib().lsa_topk_workspace_size(B, n_q, L_max, k, C.byref(nb)))
    ws = _workspace(nb.value, dev) if use_ws else None
    nbytes = nb.value if use_ws else 0
    st = lib().lsa_topk(_ptr(scores), ld, _ptr(q_pos), _ptr(kept_blocks), block_size, n_keep, B, n_q, L_max, k,
                        _ptr(idx), _ptr(count), _ptr(ws), nbytes, _stream(dev))
    _check("lsa_topk", st)
    return idx, count


def lsa_sparse_attn(q, k, v, idx, scale: Optional[float] = None, n_split: int = 0, return_lse: bool = True):
    """Sparse attention: (out bf16 [B, n_q, H_q, d], lse fp32 [B, n_q, H_q] or None).
    k, v bf16 [B, L_max, d], or pools [n_slots, d] shared by all sequences (paged caches;
    idx then holds pool rows: lsa_sparse_attn_pool)."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(idx, "idx", torch.int32, dev)
    B, n_q, H_q, d = q.shape
    pool = k.dim() == 2
    L = k.shape[0] if pool else k.shape[1]
    k_top = idx.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((B, n_q, H_q), dtype=torch.float32, device=dev) if return_lse else None
    nb = SZ(0)
    _check("lsa_sparse_attn_workspace_size",
           lib().lsa_sparse_attn_workspace_size(B, n_q, H_q, d, k_top, n_split, C.byref(nb)))
    ws = _workspace(nb.value, dev)
    fn = "lsa_sparse_attn_pool" if pool else "lsa_sparse_attn"
    st = getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), B, n_q, L, H_q, d, k_top, float(scale),
                            n_split, _ptr(out), _ptr(lse), _ptr(ws), nb.value, _stream(dev))
    _check(fn, st)
    return out, lse


# selection of flat prefill rows (lsa_forward_args.select_mode)
SELECT_MODES = {"auto": 0, "table": 1, "force_short": 2, "force_overflow": 3}
# selection of semantic decode rows (lsa_semantic_params.select_mode)
SEM_SELECT_MODES = {"row": 0, "threshold": 1, "force_short": 2, "force_overflow": 3}


def _forward_args(inp: dict, k_top: int, two_stage, block_size: int, n_keep: int, scale, attn_split: int,
                  chunk_rows: int, out: dict, select: str = "auto"):
    q_idx, k_idx, w, q_pos, q, k, v = (inp[n] for n in ("q_idx", "k_idx", "w", "q_pos", "q", "k", "v"))
    B, n_q, H_I, d_I = q_idx.shape
    _, _, H_q, d = q.shape
    pt = inp.get("page_table")
    if pt is not None:
        # paged caches: k_idx / k / v are pools [n_slots, .], keys reach them through pt
        page_size = int(inp["page_size"])
        L = pt.shape[1] * page_size
    else:
        L = k_idx.shape[1]
    a = ForwardArgs()
    a.mode = 1 if (n_q == 1 and B > 1) else 0
    # two_stage: False / True (block prefilter, then tokens) / "pooled" (kept blocks' keys)
    a.two_stage = 2 if two_stage == "pooled" else (1 if two_stage else 0)
    a.q_idx, a.k_idx, a.w = q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr()
    a.w_per_query = 1 if w.dim() == 3 else 0
    a.q_pos, a.q, a.k, a.v = q_pos.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.B, a.n_q, a.L_max, a.H_I, a.d_I, a.H_q, a.d, a.k_top = B, n_q, L, H_I, d_I, H_q, d, k_top
    a.block_size, a.n_keep = block_size, n_keep
    a.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    a.attn_split = attn_split
    a.chunk_rows = chunk_rows
    a.idx = out["idx"].data_ptr()
    a.count = out["count"].data_ptr() if out.get("count") is not None else None
    a.out = out["out"].data_ptr()
    a.lse = out["lse"].data_ptr() if out.get("lse") is not None else None
    a.kept_blocks = out["kept"].data_ptr() if out.get("kept") is not None else None
    if select not in SELECT_MODES:
        raise ValueError(f"select must be one of {sorted(SELECT_MODES)}")
    a.select_mode = SELECT_MODES[select]
    if inp.get("block_keys") is not None:
        a.block_keys = inp["block_keys"].data_ptr()
    if pt is not None:
        a.page_table = pt.data_ptr()
        a.page_size = page_size
        a.max_pages = pt.shape[1]
        a.n_slots = k_idx.shape[0]
    return a


def lsa_forward_workspace_size(inp: dict, k_top: int, two_stage=False, block_size: int = 128,
                               n_keep: int = 64, attn_split: int = 0, chunk_rows: int = 0,
                               select: str = "auto") -> int:
    dummy = {"idx": inp["q_pos"], "out": inp["q"]}
    a = _forward_args(inp, k_top, two_stage, block_size, n_keep, None, attn_split, chunk_rows, dummy, select)
    nb = SZ(0)
    _check("lsa_forward_workspace_size", lib().lsa_forward_workspace_size(C.byref(a), C.byref(nb)))
    return nb.value


def lsa_forward_plan(inp: dict, k_top: int, ws_bytes: int, two_stage=False, block_size: int = 128,
                     n_keep: int = 64, attn_split: int = 0, chunk_rows: int = 0, select: str = "auto"):
    """(rows per chunk, attention split) that lsa_forward uses with ws_bytes of workspace."""
    dummy = {"idx": inp["q_pos"], "out": inp["q"]}
    a = _forward_args(inp, k_top, two_stage, block_size, n_keep, None, attn_split, chunk_rows, dummy, select)
    rows, split = I64(0), I32(0)
    _check("lsa_forward_plan", lib().lsa_forward_plan(C.byref(a), ws_bytes, C.byref(rows), C.byref(split)))
    return rows.value, split.value


def lsa_forward_stages(inp: dict, k_top: int, ws_bytes: int, two_stage=False, block_size: int = 128,
                       n_keep: int = 64, attn_split: int = 0, chunk_rows: int = 0, select: str = "auto") -> list:
    """Names of the stages lsa_forward runs with ws_bytes of workspace, in launch order."""
    dummy = {"idx": inp["q_pos"], "out": inp["q"]}
    a = _forward_args(inp, k_top, two_stage, block_size, n_keep, None, attn_split, chunk_rows, dummy, select)
    n = I32(0)
    _check("lsa_forward_stages", lib().lsa_forward_stages(C.byref(a), ws_bytes, None, 0, C.byref(n)))
    codes = (I32 * max(n.value, 1))()
    _check("lsa_forward_stages", lib().lsa_forward_stages(C.byref(a), ws_bytes, codes, n.value, C.byref(n)))
    return [STAGE_NAMES[codes[i]] for i in range(n.value)]


def lsa_forward(inp: dict, k_top: int, two_stage=False, block_size: int = 128, n_keep: int = 64,
                scale: Optional[float] = None, attn_split: int = 0, chunk_rows: int = 0,
                out: Optional[dict] = None, ws: Optional[torch.Tensor] = None, stage_events=None,
                select: str = "auto", noalloc: bool = False) -> dict:
    """The whole path.  ``inp`` holds q_idx, k_idx, w, q_pos, q, k, v (device tensors).
    ``two_stage``: False (flat), True (block prefilter, then tokens) or "pooled" (the keys
    of the kept blocks; k_top = n_keep * block_size); ``inp["block_keys"]`` (optional,
    from lsa_block_cache) spares the block modes rebuilding the block-key cache.
    Paged caches: ``inp`` also holds page_table (int32 [B, max_pages]) and page_size;
    k_idx, k and v are then pools [n_slots, .] and idx receives pool rows.
    Returns dict(idx, count, out, lse[, kept]); pass ``out`` / ``ws`` to reuse buffers.
    ``stage_events``: optional torch.cuda.Event list (1 + len(lsa_forward_stages(...)));
    each must have been recorded once (so its HIP event exists).  ``noalloc``: run as
    lsa_forward_noalloc (the library's device array as the workspace; ``ws`` must be None)."""
    q_idx, q = inp["q_idx"], inp["q"]
    dev = q_idx.device
    for name, dt in (("q_idx", torch.int8), ("k_idx", torch.int8), ("w", torch.int32), ("q_pos", torch.int32),
                     ("q", torch.bfloat16), ("k", torch.bfloat16), ("v", torch.bfloat16)):
        _need(inp[name], name, dt, dev)
    if inp.get("page_table") is not None:
        _need(inp["page_table"], "page_table", torch.int32, dev)
    if inp.get("block_keys") is not None:
        _need(inp["block_keys"], "block_keys", torch.int8, dev)
    B, n_q = q_idx.shape[:2]
    H_q = q.shape[2]
    if out is None:
        out = {
            "idx": torch.empty((B, n_q, k_top), dtype=torch.int32, device=dev),
            "count": torch.empty((B, n_q), dtype=torch.int32, device=dev),
            "out": torch.empty_like(q),
            "lse": torch.empty((B, n_q, H_q), dtype=torch.float32, device=dev),
        }
        if two_stage:
            out["kept"] = torch.empty((B, n_q, n_keep), dtype=torch.int32, device=dev)
    a = _forward_args(inp, k_top, two_stage, block_size, n_keep, scale, attn_split, chunk_rows, out, select)
    if noalloc:
        if ws is not None:
            raise LsaError("lsa_forward_noalloc: takes no workspace")
    elif ws is None:
        nb = SZ(0)
        _check("lsa_forward_workspace_size", lib().lsa_forward_workspace_size(C.byref(a), C.byref(nb)))
        ws = _workspace(nb.value, dev)
    nbytes = 0 if ws is None else ws.numel()
    handles = None
    if stage_events is not None:
        handles = (P * len(stage_events))()
        for i, e in enumerate(stage_events):
            if not e.cuda_event:
                raise LsaError("stage_events: record each event once before passing it")
            handles[i] = e.cuda_event
        a.stage_events = C.cast(handles, P)
        a.n_stage_events = len(stage_events)
    if noalloc:
        _check("lsa_forward_noalloc", lib().lsa_forward_noalloc(C.byref(a), _stream(dev)))
    else:
        _check("lsa_forward", lib().lsa_forward(C.byref(a), _ptr(ws), nbytes, _stream(dev)))
    return out


def lsa_forward_noalloc(inp: dict, k_top: int, two_stage=False, block_size: int = 128, n_keep: int = 64,
                        scale: Optional[float] = None, attn_split: int = 0, chunk_rows: int = 0,
                        out: Optional[dict] = None, stage_events=None, select: str = "auto") -> dict:
    """lsa_forward working in the library's own device array (no workspace argument; the
    call allocates nothing -- pass ``out`` to keep torch from allocating the outputs)."""
    return lsa_forward(inp, k_top, two_stage, block_size, n_keep, scale, attn_split, chunk_rows, out=out,
                       stage_events=stage_events, select=select, noalloc=True)


# --------------------------------------------------------------------------- flat semantic search
def _sem_pages(paged: Optional[dict], cache: dict, n_slots: int = 0):
    """SemanticPages from ``paged`` = dict(block_table=int32 [B, NB] or None,
    page_table=int32 [B, max_pages] or None, page_size=int), and the logical L_max."""
    bt, pt = paged.get("block_table"), paged.get("page_table")
    P_ = int(paged.get("page_size", 0)) if pt is not None else 0
    mp = pt.shape[1] if pt is not None else 0
    nbs = cache["table"].shape[0] if bt is not None else 0
    return SemanticPages(_ptr(bt), nbs, _ptr(pt), P_, mp, n_slots if pt is not None else 0), mp * P_


def lsa_semantic_cache(k_idx, n_cluster: int = 512, n_pool: int = 4, n_bavg: int = 8, n_bmax: int = 32,
                       n_blocks: Optional[int] = None, cache: Optional[dict] = None, first_block: int = 0,
                       n_update: Optional[int] = None, paged: Optional[dict] = None,
                       n_bslots: Optional[int] = None) -> dict:
    """Bucket cache of the complete cluster blocks of k_idx (bf16 [B, L_max, 64]) through
    lsa_semantic_cluster.  With ``cache`` given, only blocks [first_block, first_block +
    n_update) are (re)clustered into it.  Returns dict(centroids bf16 [B, NB, 8, 64, 8],
    table int32 [B, NB, n_cluster], offsets int32 [B, NB, m + 1], params).

    ``paged`` (lsa_semantic_cluster_paged) = dict(block_table=int32 [B, NB] or None,
    page_table=int32 [B, max_pages] or None, page_size): with a block table the cache is a
    pool of ``n_bslots`` entries ([n_bslots, ...] arrays; NB = block_table.shape[1]); with a
    page table k_idx is the key pool [n_slots, 64] and L_max = max_pages * page_size."""
    _need(k_idx, "k_idx", torch.bfloat16)
    dev = k_idx.device
    prm = SemanticParams(n_cluster, n_pool, n_bavg, n_bmax)
    if paged is not None and paged.get("page_table") is not None:
        B, mp = paged["page_table"].shape
        L = mp * int(paged["page_size"])
        d = k_idx.shape[-1]
    else:
        B, L, d = k_idx.shape
    if paged is not None and paged.get("block_table") is not None:
        B = paged["block_table"].shape[0]
    if cache is None:
        m = n_cluster // n_bavg
        if paged is not None and paged.get("block_table") is not None:
            if n_bslots is None or n_bslots < 1:
                raise ValueError("a block-tabled cache needs n_bslots (entries of the cache pool)")
            NB = paged["block_table"].shape[1]
            lead = (n_bslots,)
        else:
            NB = L // n_cluster if n_blocks is None else n_blocks
            lead = (B, NB)
        cache = {"centroids": torch.zeros(lead + (8, 64, 8), dtype=torch.bfloat16, device=dev),
                 "table": torch.empty(lead + (n_cluster,), dtype=torch.int32, device=dev),
                 "offsets": torch.empty(lead + (m + 1,), dtype=torch.int32, device=dev),
                 "params": (n_cluster, n_pool, n_bavg, n_bmax), "NB": NB}
    else:
        prm = SemanticParams(*cache["params"])
    NB = cache.get("NB", cache["table"].shape[1])
    if n_update is None:
        n_update = min(NB, L // prm.n_cluster) - first_block
    if paged is None:
        _check("lsa_semantic_cluster",
               lib().lsa_semantic_cluster(_ptr(k_idx), B, L, d, C.byref(prm), NB, first_block, n_update,
                                          _ptr(cache["centroids"]), _ptr(cache["table"]), _ptr(cache["offsets"]),
                                          _stream(dev)))
    else:
        sp, _ = _sem_pages(paged, cache, k_idx.shape[0] if paged.get("page_table") is not None else 0)
        _check("lsa_semantic_cluster_paged",
               lib().lsa_semantic_cluster_paged(_ptr(k_idx), B, L, d, C.byref(prm), C.byref(sp), NB, first_block,
                                                n_update, _ptr(cache["centroids"]), _ptr(cache["table"]),
                                                _ptr(cache["offsets"]), _stream(dev)))
    return cache


def lsa_semantic_select(q_idx, q_pos, cache: dict, k: int, p_top: int, n_sink: int, n_w: int,
                        idx=None, count=None, ws_bytes: Optional[int] = None, ws: Optional[torch.Tensor] = None,
                        paged: Optional[dict] = None, stage_events=None, select: str = "row"):
    """Index lists of flat semantic search: (idx int32 [B, n_q, n_sink + k + n_w], count
    int32 [B, n_q]).  q_idx bf16 [B, n_q, 64]; q_pos int32 [B, n_q].  ``paged``: as for
    lsa_semantic_cache, plus n_slots (rows of the key pools) with a page table; the lists
    then hold pool rows.  ``stage_events``: three torch.cuda.Events (created and recorded
    once beforehand) recorded before and after the centroid scan and at the end
    (lsa_semantic_select_timed; contiguous caches).  ``select``: how decode rows find their
    top-p buckets (lsa_semantic_params.select_mode; a key of SEM_SELECT_MODES)."""
    _need(q_idx, "q_idx", torch.bfloat16)
    dev = q_idx.device
    _need(q_pos, "q_pos", torch.int32, dev)
    B, n_q, d = q_idx.shape
    prm = SemanticParams(*cache["params"], SEM_SELECT_MODES[select])
    NB = cache.get("NB", cache["table"].shape[1])
    W = n_sink + k + n_w
    if idx is None:
        idx = torch.empty((B, n_q, W), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    if ws is not None:
        _need(ws, "ws", torch.uint8, dev)
        ws_bytes = ws.numel()
    else:
        if ws_bytes is None:
            nb = SZ(0)
            _check("lsa_semantic_select_workspace_size",
                   lib().lsa_semantic_select_workspace_size(B, n_q, NB, C.byref(prm), C.byref(nb)))
            ws_bytes = nb.value
        ws = _workspace(ws_bytes, dev)
    if paged is None and stage_events is not None:
        evs = (P * 3)(*[C.c_void_p(e.cuda_event) for e in stage_events])
        _check("lsa_semantic_select_timed",
               lib().lsa_semantic_select_timed(_ptr(q_idx), _ptr(q_pos), B, n_q, d, C.byref(prm), NB,
                                               _ptr(cache["centroids"]), _ptr(cache["table"]),
                                               _ptr(cache["offsets"]), k, p_top, n_sink, n_w, _ptr(idx),
                                               _ptr(count), _ptr(ws), ws_bytes, _stream(dev), evs))
    elif paged is None:
        _check("lsa_semantic_select",
               lib().lsa_semantic_select(_ptr(q_idx), _ptr(q_pos), B, n_q, d, C.byref(prm), NB,
                                         _ptr(cache["centroids"]), _ptr(cache["table"]), _ptr(cache["offsets"]),
                                         k, p_top, n_sink, n_w, _ptr(idx), _ptr(count), _ptr(ws), ws_bytes,
                                         _stream(dev)))
    else:
        sp, L = _sem_pages(paged, cache, int(paged.get("n_slots", 0)))
        _check("lsa_semantic_select_paged",
               lib().lsa_semantic_select_paged(_ptr(q_idx), _ptr(q_pos), B, n_q, d, C.byref(prm), C.byref(sp), L, NB,
                                               _ptr(cache["centroids"]), _ptr(cache["table"]),
                                               _ptr(cache["offsets"]), k, p_top, n_sink, n_w, _ptr(idx),
                                               _ptr(count), _ptr(ws), ws_bytes, _stream(dev)))
    return idx, count


def lsa_semantic_workspace_size(B: int, n_q: int, cache: dict) -> int:
    """lsa_semantic_select_workspace_size for a cache of lsa_semantic_cache."""
    nb = SZ(0)
    prm = SemanticParams(*cache["params"])
    _check("lsa_semantic_select_workspace_size",
           lib().lsa_semantic_select_workspace_size(B, n_q, cache.get("NB", cache["table"].shape[1]), C.byref(prm),
                                                    C.byref(nb)))
    return nb.value


def lsa_semantic_forward(inp: dict, cache: dict, k: int, p_top: int, n_sink: int, n_w: int,
                         scale: Optional[float] = None, attn_split: int = 0, select: str = "row") -> dict:
    """Flat semantic search then sparse attention over its lists: lsa_semantic_select
    and lsa_sparse_attn.  inp: q_sem bf16 [B, n_q, 64], q_pos, q / k / v as for
    lsa_sparse_attn.  Returns dict(idx, count, out, lse)."""
    idx, count = lsa_semantic_select(inp["q_sem"], inp["q_pos"], cache, k, p_top, n_sink, n_w, select=select)
    out, lse = lsa_sparse_attn(inp["q"], inp["k"], inp["v"], idx, scale=scale, n_split=attn_split)
    return {"idx": idx, "count": count, "out": out, "lse": lse}
