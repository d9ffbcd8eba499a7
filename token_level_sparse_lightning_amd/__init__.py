"""DSA token-level sparse selection for AMD Instinct MI355X (gfx950).

The compute lives in libtlsl.so (hand-written HIP kernels behind the C ABI of
``include/tlsl.h``); this package only loads it and marshals torch tensors.
"""
from .binding import (  # noqa: F401
    BF16,
    F32,
    FP8_E4M3,
    TlslError,
    calib_copy,
    calib_mfma,
    cutoff_margin,
    dense_attn_prefill,
    dsa_prefill,
    index_decode,
    index_prefill,
    index_prefill_rerank,
    index_prefill_workspace_bytes,
    indexer_loss_grad,
    load,
    selection_quality,
    set_debug,
    sparse_attn_decode,
    sparse_attn_decode_workspace_bytes,
    sparse_attn_prefill,
    timer_arm,
    timer_collect,
    topk_select,
    topk_select_noalloc,
    topk_select_workspace_bytes,
)
