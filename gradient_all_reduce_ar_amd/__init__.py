"""MI355X-native gradient all-reduce schedules (ring, hierarchical, Rabenseifner,
recursive doubling, binary and double binary trees; fp32, bf16 and blockwise
INT8 with error feedback).

The compute path is the HIP library libar.so (csrc/), reached through the
C ABI declared in include/ar.h; this package only marshals arguments.
"""

from ._binding import (  # noqa: F401
    AR_ALLGATHER, AR_ALLREDUCE, AR_BFLOAT16, AR_BFLOAT16_EACH_STEP, AR_DOUBLE_TREE, AR_EXEC_ONEPASS, AR_EXEC_STEPS,
    AR_EXEC_STEPS_UNFUSED, AR_FLOAT32, AR_HIERARCHICAL, AR_INT8_EF, AR_RABENSEIFNER, AR_RECURSIVE_DOUBLING,
    AR_REDUCE_SCATTER, AR_RING, AR_TREE, ArError, ar_allgather, ar_allreduce, ar_allreduce_ef, ar_allreduce_noalloc, ar_bucket_allreduce, ar_bucket_allreduce_after, ar_bucket_allreduce_ef,
    ar_bucket_batched_plan, ar_bucket_count, ar_bucket_layout, ar_bucket_plan_create, ar_bucket_plan_destroy,
    ar_bucket_range, ar_bucket_set_batching, ar_bucket_set_cache_bytes, ar_bucket_set_exec, ar_bucket_set_graph,
    ar_bucket_stats, ar_last_error, ar_last_status, ar_overlap_step_time, ar_plan_cost_alpha_beta,
    ar_plan_cost_alpha_beta_ex, ar_plan_create, ar_plan_create_collective, ar_plan_destroy, ar_plan_launch_info, ar_plan_launch_ops,
    ar_plan_launch_scratch, ar_plan_launch_times, ar_plan_num_launches, ar_plan_owned_range, ar_plan_prepare,
    ar_plan_set_cache_bytes, ar_plan_set_exec, ar_plan_set_graph, ar_plan_set_profiling,
    ar_plan_set_profiling_period, ar_plan_stats, ar_plan_transfers, ar_reduce_scatter, ar_select_schedule,
)
