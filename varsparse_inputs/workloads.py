"""The synthetic workloads: shapes, scale schedules and mask parameters.

Numbers only (no method arithmetic).  Scales are 0-based indices into the
schedule; ``q_scale`` is the query scale, which attends to scales 0..q_scale.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import SCHEDULE_13, SCHEDULE_16, TINY_SIDES


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    dtype: str            # "fp32" or "bf16"
    sides: tuple
    q_scale: int
    tile: int
    n_sink: int
    radius: int           # window radius (tokens of each key scale) for every non-sink scale
    values: str           # "gaussian" or "spatial"
    budgets: tuple = field(default=())   # tile budgets of the sparsity sweep (budget mode)
    seed: int = 0
    wid: int = 0

    @property
    def radii(self):
        return [self.radius] * (self.q_scale + 1)


# Small fp32 case: 4x4-token tiles, sink = first 3 scales, window of one tile
# in mapped coordinates, read as a 4-token radius (the same mask here).
TINY = Workload("tiny_fp32", 1, 1, 64, "fp32", TINY_SIDES, 4, 4, 3, 4, "gaussian", wid=1)

# Last scale of a 2B-shaped model: 64x64 queries over 10521 cached tokens.
LAST_SCALE_2B = Workload("last_scale_2b", 2, 16, 128, "bf16", SCHEDULE_13, 12, 8, 5, 2, "spatial", wid=2)

# 8B-shaped last two scales with a budget sweep at 75/85/90/95% block sparsity.
# Budgets keep round((1 - sparsity) * nkb) tiles per query tile (floor: sinks + own tile).
LAST_TWO_8B_48 = Workload("last_two_8b_side48", 2, 28, 128, "bf16", SCHEDULE_13, 11, 8, 5, 2, "spatial",
                          budgets=(27, 16, 11, 5), wid=3)
LAST_TWO_8B_64 = Workload("last_two_8b_side64", 2, 28, 128, "bf16", SCHEDULE_13, 12, 8, 5, 2, "spatial",
                          budgets=(43, 26, 17, 9), wid=3)

# CS4A: decision scale side 32 (index 9), targets sides 40/48/64 (indices 10..12).
CS4A = Workload("cs4a_2b", 2, 16, 128, "bf16", SCHEDULE_13, 12, 8, 5, 2, "spatial", wid=4)
CS4A_DECISION = 9
CS4A_TARGETS = (10, 11, 12)
CS4A_TOP_P = 0.9

# High-resolution stress: 128x128 queries over 42521 cached tokens.
HIGH_RES = Workload("high_res_128", 1, 16, 128, "bf16", SCHEDULE_16, 15, 8, 5, 2, "spatial", wid=5)

ALL = (TINY, LAST_SCALE_2B, LAST_TWO_8B_48, LAST_TWO_8B_64, CS4A, HIGH_RES)
