"""Context-parallel sparse-attention shard for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libcsa.so`` (declared in
``include/csa.h``).  Each function has the name of its C entry point, checks
nothing itself beyond marshalling torch tensors into plain pointers and
sizes, allocates the output and workspace tensors with torch (device memory
only) and enqueues on ``torch.cuda.current_stream()``.  Every step of the
computation runs in the library's HIP kernels; when the library is missing,
importing this package raises.
"""

from ._binding import (
    Layout,
    moba_gate_topk,
    moba_gate_topk_noalloc,
    GATE_SCRATCH_BYTES,
    dsa_indexer_topk,
    sparse_attn_fwd_shard,
    sparse_attn_fwd_shard_kernel,
    sparse_attn_bwd_shard_kernel,
    sparse_attn_bwd_shard_workspace_size,
    sparse_attn_bwd_shard,
    summary_merge,
    mla_v_up_proj,
    trace_begin,
    trace_collect,
    library_path,
    lib,
    CSA_SEL_BLOCK,
    CSA_SEL_TOKEN,
    CsaError,
)

__all__ = [
    "Layout",
    "moba_gate_topk",
    "moba_gate_topk_noalloc",
    "GATE_SCRATCH_BYTES",
    "dsa_indexer_topk",
    "sparse_attn_fwd_shard",
    "sparse_attn_fwd_shard_kernel",
    "sparse_attn_bwd_shard_kernel",
    "sparse_attn_bwd_shard_workspace_size",
    "sparse_attn_bwd_shard",
    "summary_merge",
    "mla_v_up_proj",
    "trace_begin",
    "trace_collect",
    "library_path",
    "lib",
    "CSA_SEL_BLOCK",
    "CSA_SEL_TOKEN",
    "CsaError",
]
