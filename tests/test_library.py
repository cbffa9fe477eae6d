"""The C-ABI library loads and exports every symbol the headers in include/ declare (no GPU calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_calls():
    names = _declared()
    for n in ("lsa_index_scores", "lsa_block_reps", "lsa_block_prefilter", "lsa_topk", "lsa_sparse_attn",
              "lsa_forward", "lsa_forward_workspace_size", "lsa_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import learned_top_sparse_amd as lsa
    path = lsa.lib_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(lsa.EXPORTED) == _declared()
    assert lsa.lsa_version() >= 10000
    assert "INVALID" in lsa.lsa_status_string(-1)


def test_host_validation_without_gpu():
    """Invalid arguments are rejected on the host before any launch (safe without a GPU)."""
    import learned_top_sparse_amd as lsa
    L = lsa.lib()
    nb = ctypes.c_size_t(0)
    assert L.lsa_topk(None, 0, None, None, 0, 0, 1, 1, 10, 0, None, None, None, 0, None) == -1      # k < 1
    assert L.lsa_topk(None, 10, None, None, 0, 0, 1, 1, 10, 5000, None, None, None, 0, None) == -2  # k > 4096
    assert L.lsa_index_scores(None, None, None, 0, None, None, 0, 0, 1, 1, 10, 64, 96, None, 10, None) == -1
    assert L.lsa_sparse_attn(None, None, None, None, 1, 1, 10, 16, 64, 8, 1.0, 0, None, None, None, 0, None) == -2
    assert L.lsa_sparse_attn_workspace_size(64, 1, 16, 128, 2048, 0, ctypes.byref(nb)) == 0 and nb.value > 0
    assert L.lsa_block_reps(None, 1, 100, 128, 200, 1, None, None) == -2    # block_size > 128
    # zero-size work is a no-op success
    assert L.lsa_topk(None, 0, None, None, 0, 0, 0, 5, 10, 8, None, None, None, 0, None) == 0


def test_semantic_validation_without_gpu():
    """Flat semantic search: parameter checks on the host, workspace sizes, no-op calls."""
    import learned_top_sparse_amd as lsa
    L = lsa.lib()
    P = lsa.SemanticParams
    ok = P(512, 4, 8, 32)
    nb = ctypes.c_size_t(0)
    assert L.lsa_semantic_select_workspace_size(64, 1, 256, ctypes.byref(ok), ctypes.byref(nb)) == 0
    # decode rows of 16384 buckets: the score row and the threshold list (4096 entries,
    # count, threshold); prefill rows only the score row
    assert nb.value == 64 * (64 * 4 + 256 * 64 * 4 + 4096 * 8 + 8)
    assert L.lsa_semantic_select_workspace_size(1, 64, 256, ctypes.byref(ok), ctypes.byref(nb)) == 0
    assert nb.value == 64 * (64 * 4 + 256 * 64 * 4)
    for bad in (P(512, 4, 8, 15), P(512, 3, 8, 32), P(512, 4, 7, 32), P(512, 8, 4, 32), P(0, 1, 1, 2),
                P(512, 4, 8, 32, 4)):
        assert L.lsa_semantic_cluster(None, 1, 4096, 64, ctypes.byref(bad), 8, 0, 8, None, None, None, None) == -1
    assert L.lsa_semantic_cluster(None, 1, 4096, 128, ctypes.byref(ok), 8, 0, 8, None, None, None, None) == -2
    # 512 pool keys per block, or more than 64 buckets: beyond the compiled limits
    assert L.lsa_semantic_cluster(None, 1, 4096, 64, ctypes.byref(P(512, 1, 8, 32)), 8, 0, 8,
                                  None, None, None, None) == -2
    assert L.lsa_semantic_cluster(None, 1, 4096, 64, ctypes.byref(P(512, 2, 4, 8)), 8, 0, 8,
                                  None, None, None, None) == -2
    # blocks beyond the keys or the cache
    assert L.lsa_semantic_cluster(None, 1, 4000, 64, ctypes.byref(ok), 8, 0, 8, None, None, None, None) == -1
    assert L.lsa_semantic_cluster(None, 1, 4096, 64, ctypes.byref(ok), 4, 2, 3, None, None, None, None) == -1
    assert L.lsa_semantic_cluster(None, 0, 4096, 64, ctypes.byref(ok), 8, 0, 8, None, None, None, None) == 0
    sel = L.lsa_semantic_select
    assert sel(None, None, 1, 1, 64, ctypes.byref(ok), 8, None, None, None, 0, 8, 4, 512,
               None, None, None, 0, None) == -1                                       # k < 1
    assert sel(None, None, 1, 1, 64, ctypes.byref(ok), 8, None, None, None, 5000, 8, 4, 512,
               None, None, None, 0, None) == -2                                       # k > 4096
    assert sel(None, None, 1, 1, 64, ctypes.byref(ok), 8, None, None, None, 64, 4096, 4, 512,
               None, None, None, 0, None) == -2                                       # p_top > 2048
    assert sel(None, None, 0, 1, 64, ctypes.byref(ok), 8, None, None, None, 64, 16, 4, 512,
               None, None, None, 0, None) == 0                                        # nothing to do


def test_semantic_workspace_covers_span_candidates():
    """Rows that take the long-row path (more buckets than the registers hold, key
    positions beyond the largest bitmap, or buckets above 64 keys) get room for the last
    span's candidates, 2 * (2048 + 1) floats past the row's scores; other rows do not."""
    import learned_top_sparse_amd as lsa
    L = lsa.lib()
    P = lsa.SemanticParams

    def row_bytes(prm, n_blocks):
        nb = ctypes.c_size_t(0)
        assert L.lsa_semantic_select_workspace_size(1, 1, n_blocks, ctypes.byref(prm), ctypes.byref(nb)) == 0
        return nb.value

    slack = 2 * (2048 + 1)
    lst = 4096 * 8 + 8  # a decode row's threshold list, for rows of more than 4096 buckets
    up4 = lambda n: (n + 3) // 4 * 4
    # 32 buckets a block: 512 blocks put positions at the bitmap's end, 513 past it
    assert row_bytes(P(512, 4, 16, 64), 512) == 4 * 64 + 4 * 512 * 32 + lst
    assert row_bytes(P(512, 4, 16, 64), 513) == 4 * 64 + 4 * up4(513 * 32 + slack) + lst
    # 64 buckets a block: 512 blocks fill the registers, 513 exceed them
    assert row_bytes(P(512, 4, 8, 32), 512) == 4 * 64 + 4 * 512 * 64 + lst
    assert row_bytes(P(512, 4, 8, 32), 513) == 4 * 64 + 4 * up4(513 * 64 + slack) + lst
    # buckets of up to 128 keys (4 blocks: 256 buckets, no list)
    assert row_bytes(P(512, 4, 8, 128), 4) == 4 * 64 + 4 * up4(4 * 64 + slack)


def _fake_inputs(B, n_q, L, H_I=64, d_I=128, H_q=16, d=128):
    """CPU tensors with the path's shapes: only their pointers reach the host-side planning."""
    import torch
    return {
        "q_idx": torch.zeros((B, n_q, H_I, d_I), dtype=torch.int8),
        "k_idx": torch.zeros((B, L, d_I), dtype=torch.int8),
        "w": torch.ones((H_I,), dtype=torch.int32),
        "q_pos": torch.zeros((B, n_q), dtype=torch.int32),
        "q": torch.zeros((B, n_q, H_q, d), dtype=torch.bfloat16),
        "k": torch.zeros((B, L, d), dtype=torch.bfloat16),
        "v": torch.zeros((B, L, d), dtype=torch.bfloat16),
    }


def test_forward_stages_listing():
    """lsa_forward_stages: the stage sequence of each mode (host planning only)."""
    import learned_top_sparse_amd as lsa
    # decode-shaped, long rows: the indexer leaves the selection state (no score table)
    inp = _fake_inputs(64, 1, 131073)
    ws = lsa.lsa_forward_workspace_size(inp, 2048)
    assert lsa.lsa_forward_stages(inp, 2048, ws) == ["index_select", "topk", "sparse_attn"]
    # short decode rows take the decode selection as well
    inp = _fake_inputs(8, 1, 20000)
    ws = lsa.lsa_forward_workspace_size(inp, 2048)
    assert lsa.lsa_forward_stages(inp, 2048, ws) == ["index_select", "topk", "sparse_attn"]
    # ten queries in chunks of eight: the thresholded selection for the first chunk (rows
    # may be longer than 8k keys), the decode selection for the last two queries
    inp = _fake_inputs(1, 10, 40000)
    ws = lsa.lsa_forward_workspace_size(inp, 2048, chunk_rows=8)
    assert lsa.lsa_forward_stages(inp, 2048, ws, chunk_rows=8) == [
        "sample", "index_select", "topk", "sparse_attn", "index_select", "topk", "sparse_attn"]
    # ... and with the score table asked for, the table for the first chunk
    ws = lsa.lsa_forward_workspace_size(inp, 2048, chunk_rows=8, select="table")
    assert lsa.lsa_forward_stages(inp, 2048, ws, chunk_rows=8, select="table") == [
        "index_scores", "topk", "sparse_attn", "index_select", "topk", "sparse_attn"]
    # rows no longer than 8k keys keep the score table
    inp = _fake_inputs(1, 64, 16384)
    ws = lsa.lsa_forward_workspace_size(inp, 2048)
    assert lsa.lsa_forward_stages(inp, 2048, ws) == ["index_scores", "topk", "sparse_attn"]
    # prefill in three chunks (rows up to 8192 keys, k = 512: thresholded selection)
    inp = _fake_inputs(1, 3000, 8192)
    ws = lsa.lsa_forward_workspace_size(inp, 512, chunk_rows=1000)
    assert lsa.lsa_forward_stages(inp, 512, ws, chunk_rows=1000) == [
        "sample", "index_select", "topk", "sparse_attn"] * 3
    # two-stage: the block-key cache once, then per chunk the block prefilter, the token
    # stage with its top-k in one kernel (kept slots fit one workgroup), the attention
    inp = _fake_inputs(1, 512, 8192)
    ws = lsa.lsa_forward_workspace_size(inp, 512, two_stage=True, chunk_rows=256)
    st = lsa.lsa_forward_stages(inp, 512, ws, two_stage=True, chunk_rows=256)
    assert st == ["block_reps"] + ["block_prefilter", "index_select", "sparse_attn"] * 2
    # ... and with more kept slots than one workgroup holds, the token score table
    ws = lsa.lsa_forward_workspace_size(inp, 512, two_stage=True, block_size=128, n_keep=100, chunk_rows=256)
    st = lsa.lsa_forward_stages(inp, 512, ws, two_stage=True, block_size=128, n_keep=100, chunk_rows=256)
    assert st == ["block_reps"] + ["block_prefilter", "index_scores", "topk", "sparse_attn"] * 2


def test_two_stage_interleaved_key_copy_sizing():
    """Prefill-shaped two-stage forwards (every index key read at least 8 times) reserve the
    token stage's chunk-interleaved key copy -- ceil(L / 64) * 64 keys of d_I bytes per
    sequence -- in the workspace; a workspace too small for the copy plans without it (in
    chunks of the rows that fit) instead of failing; decode-shaped forwards never reserve it."""
    import learned_top_sparse_amd as lsa
    L = 20000
    il = (L + 63) // 64 * 64 * 128
    pre = _fake_inputs(1, 64, L)
    ws = lsa.lsa_forward_workspace_size(pre, 2048, two_stage=True)
    flat_blocks = lsa.lsa_forward_workspace_size(pre, 2048, two_stage=True, block_size=16, n_keep=6)  # no copy: bs % 64
    assert ws >= il
    assert lsa.lsa_forward_plan(pre, 2048, ws, two_stage=True)[0] == 64
    small = il - (1 << 16)
    assert small < ws
    rows, _ = lsa.lsa_forward_plan(pre, 2048, small, two_stage=True)
    assert 0 < rows < 64   # without the copy, in chunks
    dec = _fake_inputs(4, 1, L)
    ws_dec = lsa.lsa_forward_workspace_size(dec, 2048, two_stage=True)
    assert ws_dec < il   # per-row buffers of 4 rows and the block cache only
    assert flat_blocks > 0


def test_forward_chunks_equal_size():
    """Automatic chunking splits the rows into chunks of equal size (the last one at most
    one row per chunk short), as few as the workspace allows, instead of full chunks and
    a short tail; each planned chunk fits the workspace and an explicit chunk_rows is
    kept as given."""
    import math
    import learned_top_sparse_amd as lsa
    n, k = 1000, 2048
    inp = _fake_inputs(1, n, 20000)
    full = lsa.lsa_forward_workspace_size(inp, k)
    assert lsa.lsa_forward_plan(inp, k, full)[0] == n
    for f in (0.3, 0.45, 0.7, 0.97):
        ws = int(full * f)
        rows, _ = lsa.lsa_forward_plan(inp, k, ws)
        n_chunks = math.ceil(n / rows)
        assert rows == math.ceil(n / n_chunks), (f, rows)
        assert lsa.lsa_forward_workspace_size(inp, k, chunk_rows=rows) <= ws
        # one row more per chunk would not have saved a chunk: the most that fit needs as many
        fit = rows
        while lsa.lsa_forward_workspace_size(inp, k, chunk_rows=fit + 1) <= ws:
            fit += 1
        assert math.ceil(n / fit) == n_chunks, (f, rows, fit)
    assert lsa.lsa_forward_plan(inp, k, full, chunk_rows=333)[0] == 333


def test_block_threshold_keep_sizing():
    """Block modes reserve the thresholded keep's buffers -- per row the sampled scores
    (every (2 (n_keep - 1) // 32)-th block, 8 bytes, padded to 8 per row), threshold,
    state, count, a list of 4 n_keep (block, score) pairs and a fallback tile mark and
    list entry, plus the list's count -- only for prefill-shaped calls with rows over
    max(8 n_keep, 16384) blocks and a sampling stride of at least 16 (n_keep >= 257),
    and not with the score table asked for."""
    import learned_top_sparse_amd as lsa
    A = 256

    def al(x):
        return (x + A - 1) // A * A

    def thr_bytes(rows, n_blocks, nk):
        st = 2 * (nk - 1) // 32
        ld = ((n_blocks + st - 1) // st + 7) // 8 * 8
        cap = 4 * nk
        return (al(rows * ld * 8) + al(rows * 8) + 2 * al(rows * 4) + al(rows * cap * 4) + al(rows * cap * 8)
                + 2 * al(rows * 4) + al(4))

    pre = _fake_inputs(1, 64, 72000)
    kw = dict(two_stage="pooled", block_size=4, n_keep=300)
    auto = lsa.lsa_forward_workspace_size(pre, 1200, **kw)
    table = lsa.lsa_forward_workspace_size(pre, 1200, select="table", **kw)
    assert auto - table == thr_bytes(64, 18000, 300)
    for sel in ("force_short", "force_overflow"):
        assert lsa.lsa_forward_workspace_size(pre, 1200, select=sel, **kw) == auto
    # rows of at most 16384 blocks, sampling strides below 16, decode-shaped calls: none
    short = _fake_inputs(1, 64, 65536)
    assert (lsa.lsa_forward_workspace_size(short, 1200, **kw) ==
            lsa.lsa_forward_workspace_size(short, 1200, select="table", **kw))
    kw2 = dict(two_stage="pooled", block_size=4, n_keep=256)
    assert (lsa.lsa_forward_workspace_size(pre, 1024, **kw2) ==
            lsa.lsa_forward_workspace_size(pre, 1024, select="table", **kw2))
    dec = _fake_inputs(4, 1, 72000)
    assert (lsa.lsa_forward_workspace_size(dec, 1200, **kw) ==
            lsa.lsa_forward_workspace_size(dec, 1200, select="table", **kw))


def _fake_paged(B, n_q, max_pages, page_size, n_pages, H_I=64, d_I=128, H_q=16, d=128):
    import torch
    inp = _fake_inputs(B, n_q, 1, H_I, d_I, H_q, d)
    inp["k_idx"] = torch.zeros((n_pages * page_size, d_I), dtype=torch.int8)
    inp["k"] = torch.zeros((n_pages * page_size, d), dtype=torch.bfloat16)
    inp["v"] = torch.zeros((n_pages * page_size, d), dtype=torch.bfloat16)
    inp["page_table"] = torch.zeros((B, max_pages), dtype=torch.int32)
    inp["page_size"] = page_size
    return inp


def test_forward_paged_arguments():
    """Paged caches (host checks only): decode calls plan the decode selection and
    prefill calls the flat stages; page sizes below 64 or not powers of two, and pools
    not made of whole pages, are invalid; block modes plan their stages, and a two-stage
    call whose kept slots exceed the one-kernel token stage is unsupported."""
    import learned_top_sparse_amd as lsa
    from learned_top_sparse_amd.binding import LsaError
    inp = _fake_paged(64, 1, 2049, 64, 64 * 2049 + 100)
    ws = lsa.lsa_forward_workspace_size(inp, 2048)
    assert ws > 0
    assert lsa.lsa_forward_stages(inp, 2048, ws) == ["index_select", "topk", "sparse_attn"]
    for bad in (_fake_paged(4, 1, 16, 32, 80), _fake_paged(4, 1, 16, 96, 80)):
        with pytest.raises(LsaError, match="INVALID_ARG"):
            lsa.lsa_forward_workspace_size(bad, 256)
    bad = _fake_paged(4, 1, 16, 64, 80)
    bad["k_idx"] = bad["k_idx"][:-1]   # not whole pages
    with pytest.raises(LsaError, match="INVALID_ARG"):
        lsa.lsa_forward_workspace_size(bad, 256)
    pre = _fake_paged(1, 64, 512, 64, 600)   # 32768-key prefill rows: thresholded selection
    ws = lsa.lsa_forward_workspace_size(pre, 2048)
    assert lsa.lsa_forward_stages(pre, 2048, ws) == ["sample", "index_select", "topk", "sparse_attn"]
    two = _fake_paged(4, 1, 16, 64, 80)
    ws = lsa.lsa_forward_workspace_size(two, 256, two_stage=True)
    assert lsa.lsa_forward_stages(two, 256, ws, two_stage=True) == [
        "block_reps", "block_prefilter", "index_select", "sparse_attn"]
    ws = lsa.lsa_forward_workspace_size(two, 256, two_stage="pooled", block_size=4, n_keep=64)
    assert lsa.lsa_forward_stages(two, 256, ws, two_stage="pooled", block_size=4, n_keep=64) == [
        "block_reps", "block_prefilter", "expand", "sparse_attn"]
    with pytest.raises(LsaError, match="UNSUPPORTED"):
        lsa.lsa_forward_workspace_size(two, 256, two_stage=True, n_keep=100)


def test_forward_rejects_too_few_stage_events():
    """Too few stage events: LSA_ERR_INVALID_ARG before anything is launched."""
    import learned_top_sparse_amd as lsa
    from learned_top_sparse_amd.binding import ForwardArgs, _forward_args
    inp = _fake_inputs(4, 1, 40000)
    out = {"idx": inp["q_pos"], "out": inp["q"]}
    a = _forward_args(inp, 2048, False, 128, 64, None, 0, 0, out)
    n = ctypes.c_int32(0)
    ws = lsa.lsa_forward_workspace_size(inp, 2048)
    assert lsa.lib().lsa_forward_stages(ctypes.byref(a), ws, None, 0, ctypes.byref(n)) == 0 and n.value == 3
    handles = (ctypes.c_void_p * n.value)()   # one short of 1 + n
    a.stage_events = ctypes.cast(handles, ctypes.c_void_p)
    a.n_stage_events = n.value
    fake_ws = ctypes.c_void_p(1 << 20)   # never dereferenced: the call returns before any launch
    assert lsa.lib().lsa_forward(ctypes.byref(a), fake_ws, ws, None) == -1


def test_bench_refuses_several_gpus():
    """bench.py runs on one GPU: asked for more it exits with a message before touching a device."""
    import subprocess
    import sys
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert p.returncode == 2 and "one GPU" in p.stderr
