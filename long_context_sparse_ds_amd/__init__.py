"""Double Sparsity sparse decode attention for AMD MI355X (gfx950).

A thin Python binding over libdsparse.so (C ABI declared in include/ds.h):

    ds_calibrate_channels   offline label-channel calibration (CPU)
    ds_build_label_cache    gather the label channels of K into a compact cache (GPU)
    ds_decode_sparse_attn   one decode step: label scores, top-k select, sparse attention (GPU)

plus the decode step with the library's static device scratch as its workspace, for
callers that cannot allocate (ds_decode_sparse_attn_noalloc), the decode step for
sequences of unequal lengths (ds_decode_sparse_attn_ragged),
the decode step with K and V in pinned host memory (ds_decode_sparse_attn_offload),
decode with a hierarchical span search (ds_decode_hip_attn, its search ds_hip_search,
ds_hip_workspace_bytes, ds_hip_token_capacity),
the decode step in two phases (ds_decode_score, ds_decode_select_attend, and
ds_decode_score_ragged, ds_decode_select_attend_ragged for unequal lengths),
the decode step with the threshold rule (ds_decode_sparse_attn_threshold and its
phases ds_decode_score_threshold, ds_decode_select_attend_threshold),
its stages fed from caller buffers (ds_label_scores, ds_topk_select,
ds_select_attention, ds_sparse_attn_from_indices, ds_label_scores_positive) and
ds_decode_workspace_bytes.
"""
from ._binding import (DS_OK, DS_ERR_INVALID_ARGUMENT, DS_ERR_UNSUPPORTED, DS_ERR_WORKSPACE_TOO_SMALL, DS_ERR_HIP,
                       DS_DTYPE_F32, DS_DTYPE_BF16, DsError, LIB_PATH, lib, header_symbols, ds_last_error,
                       ds_version, ds_calibrate_channels, ds_build_label_cache, ds_decode_workspace_bytes,
                       ds_decode_is_one_pass, alloc_workspace, ds_decode_sparse_attn, ds_decode_sparse_attn_noalloc,
                       DS_NOALLOC_SCRATCH_BYTES, ds_decode_sparse_attn_ragged, ds_decode_score,
                       ds_decode_select_attend, ds_decode_score_ragged, ds_decode_select_attend_ragged,
                       ds_decode_sparse_attn_threshold, ds_decode_score_threshold, ds_decode_select_attend_threshold,
                       ds_label_scores_positive, ds_decode_sparse_attn_offload, ds_decode_hip_attn, ds_hip_search,
                       ds_hip_token_capacity,
                       ds_label_scores, ds_topk_select, ds_select_attention, ds_sparse_attn_from_indices)

__all__ = ["DS_OK", "DS_ERR_INVALID_ARGUMENT", "DS_ERR_UNSUPPORTED", "DS_ERR_WORKSPACE_TOO_SMALL", "DS_ERR_HIP",
           "DS_DTYPE_F32", "DS_DTYPE_BF16", "DsError", "LIB_PATH", "lib", "header_symbols", "ds_last_error",
           "ds_version", "ds_calibrate_channels", "ds_build_label_cache", "ds_decode_workspace_bytes",
           "ds_decode_is_one_pass", "alloc_workspace", "ds_decode_sparse_attn", "ds_decode_sparse_attn_noalloc",
           "DS_NOALLOC_SCRATCH_BYTES", "ds_decode_sparse_attn_ragged", "ds_decode_score",
           "ds_decode_select_attend", "ds_decode_score_ragged", "ds_decode_select_attend_ragged",
           "ds_decode_sparse_attn_threshold", "ds_decode_score_threshold", "ds_decode_select_attend_threshold",
           "ds_label_scores_positive", "ds_decode_sparse_attn_offload", "ds_decode_hip_attn", "ds_hip_search",
           "ds_hip_token_capacity", "ds_label_scores",
           "ds_topk_select", "ds_select_attention", "ds_sparse_attn_from_indices"]
