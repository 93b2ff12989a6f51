"""libmsa: MiniMax Sparse Attention (MSA) hot path for MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/msa.h``.  Every step of
the path runs in libmsa's HIP kernels; this module only marshals torch tensors
(device memory and streams) into pointers, sizes and strides, and turns status
codes into exceptions.  There is no CPU fallback: when ``libmsa.so`` is missing
the first call raises.

Calls (same names and meaning as the C functions):
    msa_index_score, msa_topk_blocks, msa_build_page_table, msa_topk_blocks_paged,
    msa_sparse_attn_decode, msa_sparse_attn_decode_select, msa_decode_step,
    msa_prefill_merged_workspace_size,
    msa_prefill_workspace_size,
    msa_sparse_attn_prefill, msa_sparse_attn_prefill_noalloc, msa_sparse_attn_prefill_merged,
    msa_prefill_merged_workspace_size,
    msa_lse_merge, msa_version, msa_gather_pages
Helper: empty_lse_part (partial LSEs in the C ABI's [rows][nslot][H] layout);
MSA_STEP_AUTO, MSA_STEP_ONE_LAUNCH, MSA_STEP_SEPARATE (msa_decode_step modes),
decode_step_sync_words (length of its int32 sync array)
Measured-peak probes (``include/msa_peaks.h``, not steps of the path):
    msa_peak_stream_read, msa_peak_stream_write, msa_peak_row_copy, msa_peak_mfma_bf16,
    msa_peak_mfma_bf16_random
"""
from .binding import (  # noqa: F401
    MSA_STEP_AUTO,
    MSA_STEP_ONE_LAUNCH,
    MSA_STEP_SEPARATE,
    Dims,
    MSAError,
    decode_step_sync_words,
    View,
    empty_lse_part,
    lib_path,
    load,
    msa_build_page_table,
    msa_decode_step,
    msa_gather_pages,
    msa_index_score,
    msa_lse_merge,
    msa_peak_mfma_bf16,
    msa_peak_mfma_bf16_random,
    msa_peak_row_copy,
    msa_peak_stream_read,
    msa_peak_stream_write,
    msa_prefill_merged_workspace_size,
    msa_prefill_workspace_size,
    msa_sparse_attn_decode,
    msa_sparse_attn_decode_select,
    msa_sparse_attn_prefill,
    msa_sparse_attn_prefill_merged,
    msa_sparse_attn_prefill_noalloc,
    msa_topk_blocks,
    msa_topk_blocks_paged,
    msa_version,
    view_of,
)
