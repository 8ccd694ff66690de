"""CSA2 hot path with an FP4 (E2M1 + E4M3 per 16 channels) main KV cache, for AMD MI355X.

The computation lives in libcsa2.so (hand-written HIP kernels for gfx950 behind a C ABI, see
include/csa2.h); `api` is its Python binding. Importing this package does not load the library;
the first call does, and fails loudly if it has not been built.
"""
from .api import (FULL, REINDEX, REUSE, IdxState, KVState, compress_kv, dequant_kv_fp4, hier_pool, index_scores,
                  index_scores_mxfp4, layer_args, layer_step, layer_workspace_size, prefill_n_vis,
                  quantize_kv_fp4, row_bytes, sparse_attn, sparse_attn_swa, sparse_attn_swa_prefill,
                  sparse_attn_workspace_size, topk)

__all__ = ["FULL", "REINDEX", "REUSE", "IdxState", "KVState", "compress_kv", "dequant_kv_fp4", "hier_pool", "index_scores",
           "index_scores_mxfp4", "layer_args", "layer_step", "layer_workspace_size", "prefill_n_vis",
           "quantize_kv_fp4", "row_bytes", "sparse_attn", "sparse_attn_swa", "sparse_attn_swa_prefill",
           "sparse_attn_workspace_size", "topk"]
