"""CPU oracle of the RRAttention sparse-prefill path (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never loads it.  See rr_oracle.c
for the definitions each function follows.
"""
from .oracle import (  # noqa: F401
    build, lib_path, pool_keys, stride_scores, stride_score_rows, block_scores, select, attention,
    xattn_stride_scores, xattn_block_scores, rescue_scores, union_masks,
    set_threads, get_threads, mask_from_list, list_from_mask, mask_quality, quality_metrics,
)
