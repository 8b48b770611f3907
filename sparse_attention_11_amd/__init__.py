"""MI355X-native DeepSeek Sparse Attention (DSA) forward for one context-parallel rank.

The compute path is the HIP library ``libdsa.so`` (gfx950 kernels behind a C ABI declared in
``include/dsa.h``); ``sparse_attention_11_amd.dsa`` is a thin ctypes binding to it with the
same entry-point names.  The binding is loaded on first use, so ``sparse_attention_11_amd.inputs``
(the seeded workload generator) can be imported on machines without the built library.
"""

_BINDING = (
    "dsa_abi_version", "dsa_last_error", "dsa_workspace_bytes", "dsa_indexer_scores",
    "dsa_topk_select", "dsa_indexer_topk", "dsa_sparse_attn", "dsa_forward", "dsa_forward_noalloc",
    "dsa_sparse_attn_bwd", "dsa_sparse_attn_bwd_workspace_bytes", "dsa_indexer_kl_loss_grad",
    "dsa_indexer_kl_workspace_bytes", "dsa_sparse_attn_bwd_indexer_kl",
    "dsa_sparse_attn_bwd_indexer_kl_workspace_bytes", "dsa_quantize_fp8_rows", "dsa_dense_attn",
    "Segment",
    "DsaError",
    "load_library",
)

__all__ = list(_BINDING)


def __getattr__(name):
    if name in _BINDING:
        from . import dsa
        return getattr(dsa, name)
    raise AttributeError(name)
