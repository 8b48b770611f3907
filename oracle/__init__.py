"""CPU oracle for the DeepSeek Sparse Attention (DSA) forward on one context-parallel rank.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's CPU-baseline
leg may import or call anything in this package.  The product path (the HIP library and its
Python binding) never imports it and shares no code with it.

Everything is plain NumPy in float64 on the host: slow, unblocked and written to be checked
against the source pages by eye.  See ``oracle.dsa`` for the functions and the passages they
follow.
"""

from .dsa import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3fn_decode,
    e4m3fn_encode,
    quantize_fp8_rows,
    row_windows,
    indexer_scores_row,
    indexer_scores,
    topk_row,
    topk_select,
    attention_row,
    sparse_attn,
    dsa_forward,
    attention_bwd_row,
    sparse_attn_bwd,
    indexer_kl_row,
    indexer_kl_loss_grad,
    dense_attn_row,
    dense_attn,
)
