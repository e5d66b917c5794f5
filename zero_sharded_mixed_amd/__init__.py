"""ZeRO-1/2 per-rank shard pipeline for one MI355X (gfx950).

The C ABI (include/zero_shard.h) is implemented by hand-written HIP kernels in csrc/ and
built in place into libzero_shard.so; this package exposes the same entry points over
torch device tensors.  PyTorch provides device memory and streams only.
"""
from ._binding import (EXPORTS, Z3_MAX_BUCKETS, LIB_PATH, LOSS_SCALER_BYTES, ZERO_BF16, ZERO_EHIP, ZERO_EINVAL,
                       ZERO_ENOMEM, ZERO_ERANGE, ZERO_FP16, ZERO_OK, Plan, ZeroError, lib, ptr_table,
                       read_loss_scaler, zero_adam_prepare, zero_adam_step, zero_adam_step_noalloc, zero_bucket_info,
                       zero_last_error, zero_loss_scaler, zero_loss_scaler_init, zero_loss_scaler_update,
                       zero_model_state_bytes, zero_overflow_check, zero_pack_bucket, zero_pack_bucket_check,
                       zero_param_info, zero_plan_bucket_info, zero_plan_create, zero_plan_create_grouped,
                       zero_plan_destroy, zero_plan_get_summary, zero_plan_model_state_bytes, zero_plan_param_info,
                       zero_plan_summary, zero_reduce_adam_bucket, zero_reduce_shard, zero_shard_init, zero_unpack,
                       zero_z3_step, zero_z3_layer_step)
from .step import ShardStep, Zero3Schedule

__all__ = ["EXPORTS", "Z3_MAX_BUCKETS", "LIB_PATH", "LOSS_SCALER_BYTES", "Plan", "ShardStep", "Zero3Schedule",
           "ZeroError", "lib", "ptr_table", "read_loss_scaler", "zero_adam_prepare", "zero_adam_step",
           "zero_adam_step_noalloc", "zero_bucket_info", "zero_last_error", "zero_loss_scaler",
           "zero_loss_scaler_init", "zero_loss_scaler_update", "zero_model_state_bytes", "zero_overflow_check",
           "zero_pack_bucket", "zero_pack_bucket_check", "zero_param_info", "zero_plan_bucket_info",
           "zero_plan_create", "zero_plan_create_grouped", "zero_plan_destroy", "zero_plan_get_summary",
           "zero_plan_model_state_bytes", "zero_plan_param_info", "zero_plan_summary", "zero_reduce_adam_bucket",
           "zero_reduce_shard", "zero_shard_init", "zero_unpack", "zero_z3_step", "zero_z3_layer_step",
           "ZERO_BF16", "ZERO_FP16", "ZERO_OK", "ZERO_EINVAL", "ZERO_ENOMEM", "ZERO_EHIP", "ZERO_ERANGE"]
