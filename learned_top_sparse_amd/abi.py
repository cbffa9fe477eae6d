"""ctypes declarations of liblsa.so's C ABI (include/lsa.h, include/lsa_peaks.h):
the argument structures and every exported function's signature.  Plain ctypes,
no torch, so that tools which only drive the host side (the sanitizer test) can
use it too."""
from __future__ import annotations

import ctypes as C

P = C.c_void_p
I32 = C.c_int32
I64 = C.c_int64
SZ = C.c_size_t

# every symbol the headers in include/ declare
EXPORTED = [
    "lsa_status_string", "lsa_version", "lsa_index_scores", "lsa_block_reps", "lsa_block_cache",
    "lsa_block_prefilter_workspace_size", "lsa_block_prefilter", "lsa_topk_workspace_size",
    "lsa_topk", "lsa_sparse_attn_workspace_size", "lsa_sparse_attn",
    "lsa_forward_workspace_size", "lsa_forward", "lsa_forward_plan", "lsa_forward_stages",
    "lsa_semantic_cluster", "lsa_semantic_select_workspace_size", "lsa_semantic_select",
    "lsa_semantic_cluster_paged", "lsa_semantic_select_paged", "lsa_sparse_attn_pool", "lsa_semantic_select_timed",
    "lsa_forward_noalloc", "lsa_block_cache_paged",
    "lsa_peak_sink_ints", "lsa_peak_mfma", "lsa_peak_read", "lsa_peak_gather",
]

NOALLOC_SCRATCH_BYTES = 128 << 20  # LSA_NOALLOC_SCRATCH_BYTES: lsa_forward_noalloc's device array


class ForwardArgs(C.Structure):
    _fields_ = [
        ("mode", I32), ("two_stage", I32),
        ("q_idx", P), ("k_idx", P), ("w", P), ("w_per_query", I32),
        ("q_pos", P), ("q", P), ("k", P), ("v", P),
        ("B", I32), ("n_q", I32), ("L_max", I32), ("H_I", I32), ("d_I", I32), ("H_q", I32),
        ("d", I32), ("k_top", I32), ("block_size", I32), ("n_keep", I32),
        ("scale", C.c_float), ("attn_split", I32), ("chunk_rows", I64),
        ("idx", P), ("count", P), ("out", P), ("lse", P), ("kept_blocks", P),
        ("stage_events", P), ("n_stage_events", I32),
        ("select_mode", I32),
        ("page_table", P), ("page_size", I32), ("max_pages", I32), ("n_slots", I64),
        ("block_keys", P),
    ]


class SemanticParams(C.Structure):
    """lsa_semantic_params of include/lsa.h."""
    _fields_ = [("n_cluster", I32), ("n_pool", I32), ("n_bavg", I32), ("n_bmax", I32), ("select_mode", I32)]


class SemanticPages(C.Structure):
    """lsa_semantic_pages of include/lsa.h."""
    _fields_ = [("block_table", P), ("n_bslots", I32), ("page_table", P), ("page_size", I32),
                ("max_pages", I32), ("n_slots", I64)]


def declare(L) -> None:
    """Set the argument and result types of every exported function on the CDLL L."""
    L.lsa_status_string.restype = C.c_char_p
    L.lsa_status_string.argtypes = [C.c_int]
    L.lsa_version.restype = C.c_int
    L.lsa_version.argtypes = []
    L.lsa_index_scores.argtypes = [P, P, P, I32, P, P, I32, I32, I32, I32, I32, I32, I32, P, I64, P]
    L.lsa_block_reps.argtypes = [P, I32, I32, I32, I32, I32, P, P]
    L.lsa_block_cache.argtypes = [P, I32, I32, I32, I32, I32, I32, I32, P, P]
    L.lsa_block_cache_paged.argtypes = [P, I64, P, I32, I32, I32, I32, I32, I32, I32, I32, P, P]
    L.lsa_block_prefilter_workspace_size.argtypes = [I32, I32, I32, I32, C.POINTER(SZ)]
    L.lsa_block_prefilter.argtypes = [P, P, P, I32, P, I32, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lsa_topk_workspace_size.argtypes = [I32, I32, I32, I32, C.POINTER(SZ)]
    L.lsa_topk.argtypes = [P, I64, P, P, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lsa_sparse_attn_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, C.POINTER(SZ)]
    L.lsa_sparse_attn.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, C.c_float, I32, P, P, P, SZ, P]
    L.lsa_sparse_attn_pool.argtypes = [P, P, P, P, I32, I32, I64, I32, I32, I32, C.c_float, I32, P, P, P, SZ, P]
    L.lsa_forward_workspace_size.argtypes = [C.POINTER(ForwardArgs), C.POINTER(SZ)]
    L.lsa_forward.argtypes = [C.POINTER(ForwardArgs), P, SZ, P]
    L.lsa_forward_noalloc.argtypes = [C.POINTER(ForwardArgs), P]
    L.lsa_peak_sink_ints.argtypes = [I32]
    L.lsa_peak_mfma.argtypes = [I32, I64, I32, P, P]
    L.lsa_peak_read.argtypes = [P, I64, I32, P, P]
    L.lsa_peak_gather.argtypes = [P, I64, P, I64, I32, P, P]
    L.lsa_forward_plan.argtypes = [C.POINTER(ForwardArgs), SZ, C.POINTER(I64), C.POINTER(I32)]
    L.lsa_forward_stages.argtypes = [C.POINTER(ForwardArgs), SZ, C.POINTER(I32), I32, C.POINTER(I32)]
    SP = C.POINTER(SemanticParams)
    L.lsa_semantic_cluster.argtypes = [P, I32, I32, I32, SP, I32, I32, I32, P, P, P, P]
    L.lsa_semantic_select_workspace_size.argtypes = [I32, I32, I32, SP, C.POINTER(SZ)]
    L.lsa_semantic_select.argtypes = [P, P, I32, I32, I32, SP, I32, P, P, P, I32, I32, I32, I32, P, P, P, SZ, P]
    L.lsa_semantic_select_timed.argtypes = [P, P, I32, I32, I32, SP, I32, P, P, P, I32, I32, I32, I32, P, P, P,
                                             SZ, P, C.POINTER(P)]
    SG = C.POINTER(SemanticPages)
    L.lsa_semantic_cluster_paged.argtypes = [P, I32, I32, I32, SP, SG, I32, I32, I32, P, P, P, P]
    L.lsa_semantic_select_paged.argtypes = [P, P, I32, I32, I32, SP, SG, I32, I32, P, P, P, I32, I32, I32, I32,
                                             P, P, P, SZ, P]
    for name in EXPORTED:
        if name not in ("lsa_status_string", "lsa_version"):
            getattr(L, name).restype = C.c_int
