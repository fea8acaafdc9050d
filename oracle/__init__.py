"""CPU oracle for the HARD-KV decode step.

Test infrastructure only: imported by the test-suite, by the package
``smoke()`` check and by the benchmark's ``cpu_baseline`` leg, never by the
product path.  It shares no code with the HIP library.
"""
from .hardkv_oracle import (  # noqa: F401
    METRIC_QK, METRIC_L2, METRIC_WINDOW, window_score_head, aged_count, score_head, calibrate_head, topp_head,
    condense, attend_head, full_attention, step_head, step, HeadState,
    init_state, lifecycle_step, POLICY_REWRITE, POLICY_SPARSE, POLICY_MTI,
    MODE_REWRITE, MODE_SPARSE, mti_head, plan_head, reuse_head, MERGE_MEAN,
    MERGE_WEIGHTED, MERGE_FLOOR, merge_weights, candidate_range, dense_positions,
    pack_heads, tier_alloc, CALIB_SPREAD, CALIB_ENTROPY, ENTROPY_STEPS, ENTROPY_SPAN, softmax_entropy,
    entropy_temperature, HeadResult, METRIC_KEYDIFF, AUX_METRICS, keydiff_head,
    METRIC_RKV, redundancy_head, block_topp_head, BlockSelection, Selection,
)
