"""DeepSeek Sparse Attention (DSA) hot path for AMD Instinct MI355X (gfx950).

Lightning Indexer scores (FP8 MFMA) -> top-k selection (LDS radix select)
-> sparse MLA over the selected latent rows (bf16 MFMA, online softmax),
plus the page-64 indexer key cache and token-granular latent KV cache
stores.  The computation lives in hand-written HIP kernels behind the C ABI
of include/dsa.h (libdsa.so); this package is the Python binding of that
ABI, with the same names.
"""
from ._binding import (  # noqa: F401
    DSAError, lib, abi_version, indexer_cache_store, kv_cache_store, cache_store, indexer_scores, topk, topk_static,
    topk_workspace_size, indexer_topk, indexer_topk_workspace_size,
    sparse_mla_prefill, sparse_mla_decode, sparse_mla_decode_workspace_size, LIB_PATH, PAGE, DK, DV,
    KV_BF16, KV_FP8_E4M3,
)
from .pipeline import prefill_step, decode_step  # noqa: F401
