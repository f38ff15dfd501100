"""Oracle of the capacity constraint and the greedy per-operation planner.

Capacity (walkthrough, section on why offloading is more than "move it to the
CPU"): with M bytes of weights and KV and H bytes of usable HBM, the global
ratio must satisfy x_global >= max(0, (M - H) / M).

Planner (DAK paper §4.2.2 "Optimal Greedy Offload"; App. A eq. 1): distribute
the budget sum_i C_i x_i = R sum_i C_i so that sum_i T_i is minimal, in three
phases:
  1. memory-bound ops, up to the end of their decreasing region;
  2. then every op, up to its turning point (the end of its flat region);
  3. then every op, up to all of it.

Discrete reading used here (units are tile-rows or requests):
  * op i has n_i units of u_i bytes and a compute time T_comp,i;
  * T_i(h) = max(T_comp,i, (n_i - h) u_i / B_g, h u_i / B_h) for h = 0..n_i;
  * a_i = smallest h minimising T_i, b_i = largest such h;
  * op i is memory-bound iff T_i(0) > T_comp,i;
  * W = ceil(R * sum_i C_i) bytes must go to the host (R times the total in
    double, then rounded up);
  * within a phase ops are visited in index order and each takes only the units
    still needed, ceil((W - S) / u_i); allocation stops once S >= W;
  * if S < W after phase 3 the request is infeasible.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

from .cost_model import unit_time


class Infeasible(ValueError):
    """The host budget cannot be met even with every unit on the host."""


@dataclass(frozen=True)
class Op:
    units: int        # n_i: tile-rows (linear) or requests (attention)
    unit_bytes: int   # u_i: bytes per unit
    t_comp: float     # T_comp,i in seconds

    @property
    def bytes(self) -> int:
        return self.units * self.unit_bytes


def min_offload_ratio(footprint: int, hbm: int) -> float:
    """Lower bound on the global ratio: max(0, (M - H) / M)."""
    if footprint <= 0:
        return 0.0
    return max(0.0, (footprint - hbm) / footprint)


def required_host_bytes(x_global: float, total_bytes: int) -> int:
    """W = ceil(x_global * total) evaluated in double."""
    if not (0.0 <= x_global <= 1.0):
        raise ValueError("x_global must lie in [0, 1]")
    return int(math.ceil(float(x_global) * float(total_bytes)))


def op_times(op: Op, b_g: float, b_h: float):
    return [unit_time(op.units, op.unit_bytes, h, op.t_comp, b_g, b_h) for h in range(op.units + 1)]


def argmin_range(op: Op, b_g: float, b_h: float):
    """(a_i, b_i): the first and the last h at which T_i(h) is minimal."""
    ts = op_times(op, b_g, b_h)
    tmin = min(ts)
    idx = [h for h, t in enumerate(ts) if t == tmin]
    return idx[0], idx[-1]


def memory_bound(op: Op, b_g: float, b_h: float) -> bool:
    return unit_time(op.units, op.unit_bytes, 0, op.t_comp, b_g, b_h) > op.t_comp


def greedy_plan(ops, b_g: float, b_h: float, W: int):
    """Host units per op for a budget of W bytes (three-phase greedy)."""
    h = [0] * len(ops)
    S = 0
    ranges = [argmin_range(op, b_g, b_h) for op in ops]
    mem = [memory_bound(op, b_g, b_h) for op in ops]

    def take(i: int, target: int) -> None:
        nonlocal S
        if S >= W or target <= h[i]:
            return
        u = ops[i].unit_bytes
        need = -(-(W - S) // u)
        add = min(target - h[i], need)
        h[i] += add
        S += add * u

    for i in range(len(ops)):          # phase 1: memory-bound ops to the end of their descent
        if mem[i]:
            take(i, ranges[i][0])
    for i in range(len(ops)):          # phase 2: every op to its turning point
        take(i, ranges[i][1])
    for i in range(len(ops)):          # phase 3: anything, up to the whole op
        take(i, ops[i].units)
    if S < W:
        raise Infeasible(f"budget {W} B exceeds the {S} B the ops hold")
    return h


def modeled_time(ops, h, b_g: float, b_h: float) -> float:
    """sum_i T_i(h_i), accumulated in op order."""
    t = 0.0
    for op, hi in zip(ops, h):
        t += unit_time(op.units, op.unit_bytes, hi, op.t_comp, b_g, b_h)
    return t


def plan(ops, b_g: float, b_h: float, x_global: float):
    """(host units per op, modelled time) for a global ratio x_global."""
    total = sum(op.bytes for op in ops)
    W = required_host_bytes(x_global, total)
    h = greedy_plan(ops, b_g, b_h, W)
    return h, modeled_time(ops, h, b_g, b_h)


def uniform_plan(ops, x_global: float):
    """Baseline of DAK §4.2.1: every op offloads the same ratio (rounded up per op)."""
    return [int(math.ceil(float(x_global) * op.units)) for op in ops]
