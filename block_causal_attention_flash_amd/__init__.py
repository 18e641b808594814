"""Block-causal QK-RMSNorm GQA attention forward for MI355X (gfx950), with the
text cross-attention that runs beside it in each transformer block.

Thin Python binding over the C ABI of libmagi_attn.so (include/magi_attn.h).
Every function has the name of the C entry point it marshals; all of the
computation runs in the HIP kernels. torch supplies device memory and streams.
"""
from .api import (CrossPlan, CrossTrainPlan, MagiAttnError, ParallelPlan, Plan, TrainPlan, magi_attn_abi_version, magi_attn_bwd,
                  magi_attn_bwd_workspace_size, magi_attn_classify_host, magi_attn_key_classify_host,
                  magi_attn_cross_train_plan_create, magi_attn_train_plan_create,
                  magi_attn_cross_classify_host, magi_attn_cross_plan_create, magi_attn_cross_plan_stats,
                  magi_attn_fwd, magi_attn_fwd_noalloc, magi_attn_fwd_parallel, magi_attn_fwd_simple, magi_attn_parallel_plan_create,
                  magi_attn_plan_create, magi_attn_plan_destroy, magi_attn_plan_stats, magi_attn_workspace_size)

__all__ = ["CrossPlan", "CrossTrainPlan", "MagiAttnError", "ParallelPlan", "Plan", "TrainPlan", "magi_attn_abi_version", "magi_attn_bwd",
           "magi_attn_bwd_workspace_size", "magi_attn_classify_host", "magi_attn_key_classify_host",
           "magi_attn_cross_train_plan_create", "magi_attn_train_plan_create",
           "magi_attn_cross_classify_host", "magi_attn_cross_plan_create", "magi_attn_cross_plan_stats",
           "magi_attn_fwd", "magi_attn_fwd_noalloc", "magi_attn_fwd_parallel", "magi_attn_fwd_simple", "magi_attn_parallel_plan_create",
           "magi_attn_plan_create", "magi_attn_plan_destroy", "magi_attn_plan_stats", "magi_attn_workspace_size"]
