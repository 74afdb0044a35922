"""CPU oracle of the quantised GEMV / expert-MLP path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  It is independent of the HIP
path: it shares no code with it and neither imports the other.  Inputs come
from the ``synth`` generators; the arithmetic is in ``oracle.c``.
"""
from .oracle import (OracleLib, load, dequant, code_values, gemv, gate_up, expert_group,
                     expert_group_down, route,
                     e2m1, minifloat, silu, set_threads, get_threads, round_fmt, v4_block_scale,
                     v4_combine, expert_group_v4)

__all__ = ["OracleLib", "load", "dequant", "code_values", "gemv", "gate_up", "expert_group",
           "expert_group_down", "route",
           "e2m1", "minifloat", "silu", "set_threads", "get_threads", "round_fmt", "v4_block_scale",
           "v4_combine", "expert_group_v4"]
