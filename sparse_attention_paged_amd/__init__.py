"""Top-k sparse attention over a paged KV cache for AMD MI355X (gfx950).

The compute lives in libsap.so (hand-written HIP kernels behind the C ABI of
include/sap.h).  This package only marshals torch device tensors into that
ABI: pointers, strides, dtypes and the current HIP stream.
"""
from ._lib import LIB_PATH, SapError, lib, status_string
from .api import (build_sparse_idx, debug_e4m3_table, debug_e4m3_f16_table, debug_fp4_table, gated_pool, indexer_logits_candidates,
                  indexer_logits_packed, indexer_logits_prefill,
                  sparse_attn_noalloc_max_bytes, sparse_attn_num_splits, sparse_attn_paged,
                  sparse_attn_paged_noalloc, sparse_attn_workspace_bytes,
                  topk_select, topk_sparse_idx, topk_workspace_bytes)

__all__ = [
    "LIB_PATH", "SapError", "lib", "status_string", "build_sparse_idx", "sparse_attn_paged",
    "sparse_attn_num_splits", "sparse_attn_workspace_bytes",
    "sparse_attn_paged_noalloc", "sparse_attn_noalloc_max_bytes", "indexer_logits_packed",
    "indexer_logits_candidates", "indexer_logits_prefill", "topk_select",
    "topk_workspace_bytes", "topk_sparse_idx", "gated_pool", "debug_e4m3_table", "debug_e4m3_f16_table", "debug_fp4_table",
]
