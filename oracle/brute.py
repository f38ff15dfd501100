"""Exhaustive search over per-op host-unit counts (DAK paper App. A, eq. 1).

Minimises sum_i T_i(h_i) over every integer plan whose host bytes S satisfy
W <= S < W + max_i u_i: the budget is met and overshot by less than one unit,
which always contains the greedy plan.  With equal unit sizes and W a multiple
of the unit this is exactly App. A's equality constraint.  Only for tiny op sets.
"""
from __future__ import annotations

import itertools

from .cost_model import unit_time


def best_plans(ops, b_g: float, b_h: float, W: int):
    """(minimal objective, list of plans attaining it)."""
    umax = max(op.unit_bytes for op in ops)
    best = None
    arg = []
    for h in itertools.product(*[range(op.units + 1) for op in ops]):
        S = sum(hi * op.unit_bytes for hi, op in zip(h, ops))
        if S < W or S >= W + umax:
            continue
        t = 0.0
        for op, hi in zip(ops, h):
            t += unit_time(op.units, op.unit_bytes, hi, op.t_comp, b_g, b_h)
        if best is None or t < best:
            best, arg = t, [list(h)]
        elif t == best:
            arg.append(list(h))
    return best, arg
