"""DSA sparse-attention layer (lightning indexer -> exact top-k -> sparse MLA) for MI355X.

The compute lives in libdsa.so (HIP kernels for gfx950 behind the C ABI of include/dsa.h); this
package is its Python binding plus a small driver that runs the three steps on one stream.
Source of the method: "vLLM Delivers Day-0 Support for Kimi K3.1 Pro", §Sparse Attention in K3.1
Pro.
"""
from ._lib import (DSAError, DeviceBatch, KVLayout, kv_layout, dsa_indexer_scores, dsa_topk,
                   dsa_topk_workspace_bytes,
                   sparse_mla_decode, sparse_mla_prefill, sparse_mla_workspace_bytes, lib,
                   IKEY_FP8, IKEY_MXFP4, LATENT_FP8, LATENT_NVFP4, MAX_TOPK, HIST_BINS,
                   MAX_ROWS_PER_SEQ, INDEX_HEADS, INDEX_DIM, MLA_HEADS, MLA_DQK, MLA_DV, EXPORTS,
                   BATCH_INVARIANT, dsa_cache_append, dsa_quantize_query, dsa_indexer_front,
                   dsa_dcp_mailbox_bytes,
                   dsa_dcp_publish, dsa_dcp_merge, dsa_lse_combine, dsa_dcp_partials_bytes,
                   sparse_mla_decode_shard, MERGE_PACKED, MERGE_SCORES,
                   MERGE_GENERIC, MAX_SHARDS, dsa_device_status, DEVERR_ROWS_PER_SEQ,
                   DEVERR_BLOCK_ID, DEVERR_POOL_ROW, sparse_mla_decode_noalloc,
                   DEVERR_CAND_OVERFLOW, dsa_candidates_workspace_bytes, dsa_indexer_candidates,
                   dsa_topk_candidates, BATCH_PLAIN_ORDER)
from .layer import DSALayer

__all__ = ["DSAError", "DeviceBatch", "KVLayout", "kv_layout", "dsa_indexer_scores", "dsa_topk", "dsa_topk_workspace_bytes",
           "sparse_mla_decode", "sparse_mla_prefill", "sparse_mla_workspace_bytes", "lib",
           "DSALayer", "EXPORTS", "BATCH_INVARIANT", "dsa_cache_append", "dsa_quantize_query",
           "dsa_indexer_front",
           "dsa_dcp_mailbox_bytes", "dsa_dcp_publish", "dsa_dcp_merge", "dsa_lse_combine",
           "dsa_dcp_partials_bytes", "sparse_mla_decode_shard",
           "MERGE_PACKED", "MERGE_SCORES", "MERGE_GENERIC", "MAX_SHARDS", "dsa_device_status",
           "DEVERR_ROWS_PER_SEQ", "DEVERR_BLOCK_ID", "DEVERR_POOL_ROW",
           "sparse_mla_decode_noalloc", "DEVERR_CAND_OVERFLOW", "dsa_candidates_workspace_bytes",
           "dsa_indexer_candidates", "dsa_topk_candidates", "BATCH_PLAIN_ORDER"]
