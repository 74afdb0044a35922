"""Quantised GEMV and expert-MLP kernels for AMD Instinct MI355X (gfx950).

The work happens in libdqg.so (hand-written HIP kernels behind the C ABI of
include/dqg.h); this package is its Python binding.
"""
from ._lib import (DQG_I3_G64, DQG_I4_GS, DQG_I4_ROW, DQG_I8_ROW, DQG_MXFP4, DQG_F32, DQG_BF16, DQG_FP8_BLOCK,
                   DQG_I8_GS, DQG_F16, DQG_ROUTE_SIGMOID,
                   DQG_ROUTE_SOFTMAX, DQG_ACT_SWIGLU, DQG_ACT_SWIGLU_V4, DqgError, Expert,
                   ExpertTable, Matrix, dqg_dequant, dqg_expert_group, dqg_expert_group_issue, dqg_expert_group_noalloc,
                   dqg_expert_group_take, dqg_gate_up, dqg_gate_up_clamped, dqg_last_error, dqg_matmul, dqg_prof_begin,
                   dqg_prof_begin_sampled, dqg_prof_end, dqg_prof_end_launches, dqg_read_bytes, dqg_route, dqg_stats, dqg_stats_reset, load)

__all__ = ["DQG_I3_G64", "DQG_I4_GS", "DQG_I4_ROW", "DQG_I8_ROW", "DQG_MXFP4", "DQG_F32", "DQG_BF16",
           "DQG_FP8_BLOCK", "DQG_I8_GS", "DQG_F16", "DQG_ROUTE_SIGMOID", "DQG_ACT_SWIGLU", "DQG_ACT_SWIGLU_V4",
           "DQG_ROUTE_SOFTMAX", "DqgError", "Expert",
           "ExpertTable", "Matrix", "dqg_dequant", "dqg_expert_group", "dqg_expert_group_issue", "dqg_expert_group_noalloc",
           "dqg_expert_group_take", "dqg_gate_up", "dqg_gate_up_clamped", "dqg_last_error", "dqg_matmul", "dqg_prof_begin",
           "dqg_prof_begin_sampled", "dqg_prof_end", "dqg_prof_end_launches", "dqg_read_bytes", "dqg_route", "dqg_stats",
           "dqg_stats_reset", "load"]
