"""MI355X-native DeepSeek Sparse Attention (DSA) forward path.

The compute lives in libdsa.so (hand-written HIP for gfx950 behind the C ABI in
include/dsa.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    BF16, F32, FP8_E4M3, LIB_PATH, NOALLOC_SCRATCH_BYTES, DsaError, DsaShape, forward, forward_min_workspace_size,
    forward_noalloc,
    forward_workspace_size, index_cache_append_fp8, index_scores, index_topk, index_topk_min_workspace_size,
    index_topk_workspace_size, lib, mla_kv_quant_fp8, rotate_quant_fp8,
    sparse_mla_bwd, sparse_mla_bwd_min_workspace_size, sparse_mla_bwd_workspace_size, sparse_mla_fwd,
    sparse_mla_workspace_size, topk, topk_workspace_size,
)
