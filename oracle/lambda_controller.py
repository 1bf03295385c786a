"""fp64 CPU oracle for the adaptive load-balancing weight (test infrastructure only).

Adaptive-lambda commit page ("2d0e6b6bdc"), formula block:
    lambda_eff = lambda_floor + lambda_max_extra * max(0, ent_target - ent_ema) / ent_target
with ent_target = entropy_target_frac * ln(K) for K experts (config knobs block: floor 0.01,
max extra 0.09, target fraction 0.7; bootstrap block: lambda starts at the floor and the
entropy EMA at ln K).  The producer of ent_ema (which entropy, which decay) is not given on
the pages; this module takes ent_ema as an input.
"""
from __future__ import annotations

import math

FLOOR, MAX_EXTRA, TARGET_FRAC = 0.01, 0.09, 0.7


def entropy_target(K: int, target_frac: float = TARGET_FRAC) -> float:
    return target_frac * math.log(K)


def lambda_eff(ent_ema: float, K: int, floor: float = FLOOR, max_extra: float = MAX_EXTRA,
               target_frac: float = TARGET_FRAC) -> float:
    target = entropy_target(K, target_frac)
    deficit = max(0.0, target - ent_ema)
    return floor + max_extra * deficit / target
