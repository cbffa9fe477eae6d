"""The C-ABI library loads and exports every symbol include/lsa.h declares (no GPU calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", src)))


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
