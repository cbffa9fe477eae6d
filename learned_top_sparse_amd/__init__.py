"""Learned top-k sparse attention for MI355X: thin Python binding of liblsa.so.

Every step of the path runs in the HIP kernels behind the C ABI of
``include/lsa.h``; this module only checks tensors, allocates outputs and
workspaces with torch (device memory and streams are all torch is used for)
and passes raw pointers plus the current HIP stream.  There is no fallback:
if ``liblsa.so`` is missing the calls raise.
"""
from .binding import (  # noqa: F401
    LsaError,
    lib,
    lib_path,
    lsa_block_cache,
    lsa_block_prefilter,
    lsa_block_reps,
    lsa_forward,
    lsa_forward_noalloc,
    NOALLOC_SCRATCH_BYTES,
    lsa_forward_plan,
    lsa_forward_stages,
    lsa_forward_workspace_size,
    lsa_index_scores,
    lsa_semantic_cache,
    lsa_semantic_forward,
    lsa_semantic_select,
    lsa_semantic_workspace_size,
    SemanticParams,
    lsa_sparse_attn,
    lsa_status_string,
    lsa_topk,
    lsa_version,
    EXPORTED,
    STAGE_NAMES,
)
