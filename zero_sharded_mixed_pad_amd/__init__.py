"""Per-rank hot path of ZeRO-3 intra-layer partitioning on MI355X (gfx950).

Each parameter is flattened, padded to a multiple of N_d and split into N_d
contiguous 1D shards; gradients of N_d virtual ranks are reduced into the
owned shard in fixed rank order (fp32); a fused mixed-precision Adam step
updates the fp32 master and moments and writes the bf16 working copy; a full
parameter is gathered and unpadded from its N_d shards just before compute.
All work runs in the HIP kernels of libzsp.so behind the C ABI in
include/zsp.h; this package is its thin ctypes binding.
"""
from .binding import (  # noqa: F401
    ALL_RANKS, BF16, F32, GRADS_FULL, GRADS_SHARD, MAX_RANKS, SRC_ACC, SRC_MASTER, SRC_WORK,
    GatherList, Plan, Schedule,
    ZspError, last_error, partition, zsp_adam_step, zsp_bind_state, zsp_checkpoint_load,
    zsp_checkpoint_read_host, zsp_checkpoint_save, zsp_checkpoint_write_host, zsp_destroy, zsp_gather,
    zsp_gather_list_create, zsp_gather_list_destroy, zsp_gather_list_run,
    zsp_gather_many, zsp_gather_many_noalloc, zsp_gather_range, zsp_load_params, zsp_partition,
    zsp_plan_info, zsp_plan_tensor,
    zsp_reduce_adam_step, zsp_reduce_adam_step_params, zsp_reduce_shard,
    zsp_reduce_shard_params, zsp_adam_step_params, zsp_sched_acquire, zsp_sched_bind, zsp_sched_create,
    zsp_sched_destroy, zsp_sched_info, zsp_sched_release, zsp_sched_reset, zsp_sched_set_engine,
)
