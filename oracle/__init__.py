"""CPU oracle for the Double Sparsity decode step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU baseline leg, never by the product path.  Every function is
pinned by a CPU test against something other than itself (closed forms,
brute force on tiny inputs, a library routine, invariants, hand-worked
fixtures); none is "parity unpinned".
"""
from .ds_oracle import (calibrate_channels, label_rows, label_scores, block_scores, select_topk,
                        blocks_to_tokens, attention_weights, attend, attend_partial, merge_partials,
                        default_scale, decode_unit, tokens_of, label_scores_positive, select_threshold,
                        decode_unit_threshold, group_token_scores, hip_search, spans_to_tokens, decode_unit_hip)

__all__ = ["calibrate_channels", "label_rows", "label_scores", "block_scores", "select_topk",
           "blocks_to_tokens", "attention_weights", "attend", "attend_partial", "merge_partials",
           "default_scale", "decode_unit", "tokens_of", "label_scores_positive", "select_threshold",
           "decode_unit_threshold", "group_token_scores", "hip_search", "spans_to_tokens", "decode_unit_hip"]
