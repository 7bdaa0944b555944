"""Dynamic sparse attention for the long-context prefill phase on MI355X.

Vertical-slash, block-sparse and streaming (A-shape) heads, each as online
sparse-index estimation followed by exact block-sparse attention (per pattern,
or a whole mixed layer with one attention launch), the KV-retention scores
and kept keys that follow prefill, sparse decode, and multi-stage
hierarchical chunk pruning (for decode rows, or as a block estimator), all in
HIP kernels for gfx950 behind a C ABI (include/dsa.h). This package is the
thin Python binding of that library; torch supplies device memory and
streams.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    DsaError,
    block_sparse_attention,
    block_sparse_workspace_bytes,
    bs_pool,
    bs_select,
    chunks_to_keys,
    hier_block_sparse_attention,
    hier_prune,
    hier_sparse_decode,
    kv_retention,
    load,
    mixed_sparse_attention,
    mixed_workspace_bytes,
    sparse_attention_blocks,
    sparse_attention_mixed,
    sparse_attention_vs,
    sparse_decode,
    sparse_decode_noalloc,
    streaming_attention,
    topk,
    vertical_slash_sparse_attention,
    vertical_slash_workspace_bytes,
    vs_build_index,
    vs_estimate,
)
