"""MI355X-native RRAttention sparse prefill.

The compute lives in librr.so (hand-written HIP kernels for gfx950 behind the
C ABI of include/rr.h); :mod:`long_context_prefill_rr_amd.rr` marshals torch
tensors into those calls.  Importing the binding fails loudly when librr.so
is missing: there is no fallback path.
"""
from .rr import (  # noqa: F401
    RRError, lib_path, load_library, rr_estimate, rr_select, rr_sparse_attn, rr_prefill,
    rr_prefill_noalloc, noalloc_scratch_bytes,
    rr_mask_quality, quality_summary, rr_xattn_estimate, rr_rescue_estimate, rr_merge_masks,
    rr_estimate_materialized, stride_scores_count,
    workspace_bytes, estimate_workspace_bytes, sparse_attn_workspace_bytes, prefill_workspace_bytes,
    rescue_workspace_bytes,
    RR_OUT_BF16, RR_OUT_F32,
)
