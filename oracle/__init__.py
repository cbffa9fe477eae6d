"""CPU oracle for the indexer -> exact top-k -> sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables
or helpers with the HIP library or its binding; the only module both sides see
is ``synthetic`` (random draws, no arithmetic of the method).

Everything here is the plain definition, computed slowly in numpy:
integer scores in int64, attention in fp64.  See ``lsa_oracle`` for the
passages each function follows.
"""
from .lsa_oracle import (  # noqa: F401
    index_scores,
    block_reps,
    block_scores,
    block_keep,
    two_stage_candidates,
    topk,
    sparse_attention,
    forward_row,
    paged_rows,
    forward_row_paged,
    sem_bf16,
    sem_normalize,
    sem_pool_keys,
    sem_ward_costs,
    sem_ward,
    sem_cluster_block,
    bucket_cache,
    sem_scores,
    sem_order_key,
    sem_top_buckets,
    sem_expand,
    semantic_select_row,
    semantic_forward_row,
)
