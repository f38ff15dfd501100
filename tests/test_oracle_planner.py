"""Pins of the capacity bound and the greedy planner (DAK paper §4.2.2 "Optimal
Greedy Offload", App. A Theorems 1-3; walkthrough capacity section; Fig. 4,
Fig. 10 and Fig. 14 tables)."""
import json
import math
import os
import random

import pytest

from oracle import planner as op
from oracle import brute, cost_model as cm
from conftest import GOLDEN


def test_capacity_ratio_reproduces_printed_tables():
    with open(os.path.join(GOLDEN, "capacity_ratios.json")) as f:
        g = json.load(f)
    H = g["hbm_bytes"]
    for r in g["rows"]:
        M = (r["weights_gb"] + r["kv_gb"]) * 1e9
        got = 100 * op.min_offload_ratio(int(M), int(H))
        assert abs(got - r["ratio_pct"]) <= g["tolerance_points"], r


def test_capacity_ratio_fig4():
    with open(os.path.join(GOLDEN, "fig4_overview.json")) as f:
        g = json.load(f)
    got = op.min_offload_ratio(int(g["footprint_bytes"]), int(g["hbm_bytes"]))
    assert 100 * got == pytest.approx(g["total_ratio_pct"], abs=1e-9)
    assert op.min_offload_ratio(100, 200) == 0.0
    assert op.min_offload_ratio(0, 5) == 0.0


def test_required_bytes_rounds_up():
    assert op.required_host_bytes(0.0, 1000) == 0
    assert op.required_host_bytes(1.0, 1000) == 1000
    assert op.required_host_bytes(0.0011, 1000) == 2
    with pytest.raises(ValueError):
        op.required_host_bytes(-0.1, 10)


def _random_ops(rng, n_ops, dyadic):
    ops = []
    for _ in range(n_ops):
        n = rng.randint(1, 6)
        if dyadic:
            u = 1 << rng.randint(2, 5)
            tc = rng.randint(0, 40) / 8.0
        else:
            u = rng.randint(1, 9)
            tc = rng.random() * 6.0
        ops.append(op.Op(n, u, tc))
    return ops


def _kink_aligned(ops, bg, bh):
    # Every per-unit marginal of T_i is -u/B_g, 0 or +u/B_h: kinks fall on units.
    u0 = ops[0].unit_bytes
    if any(o.unit_bytes != u0 for o in ops):
        return False
    for o in ops:
        ts = op.op_times(o, bg, bh)
        for a, b in zip(ts, ts[1:]):
            if b - a not in (-o.unit_bytes / bg, 0.0, o.unit_bytes / bh):
                return False
    return True


def test_greedy_equals_brute_force_on_kink_aligned_sets():
    rng = random.Random(11)
    checked = 0
    for _ in range(4000):
        bg, bh = 2.0 ** rng.randint(1, 3), 2.0 ** rng.randint(-1, 1)
        ops = _random_ops(rng, rng.randint(1, 4), dyadic=True)
        if not _kink_aligned(ops, bg, bh):
            continue
        u = ops[0].unit_bytes
        total_units = sum(o.units for o in ops)
        W = u * rng.randint(0, total_units)
        h = op.greedy_plan(ops, bg, bh, W)
        assert sum(hi * o.unit_bytes for hi, o in zip(h, ops)) == W
        best, plans = brute.best_plans(ops, bg, bh, W)
        assert op.modeled_time(ops, h, bg, bh) == best
        assert h in plans
        checked += 1
    assert checked > 200


def test_greedy_gap_on_general_tiny_sets_is_bounded_by_partial_units():
    """App. A proves the greedy optimal for real-valued ratios.  With whole units
    each op's descent end and turning point may fall inside a unit, so the
    greedy can misplace less than one unit of bytes per op at each boundary
    (each misplaced byte costs at most 1/B_g + 1/B_h), and the last unit may
    overshoot the budget.  Hence
        greedy - optimum <= (sum_i u_i + max_i u_i) * (1/B_g + 1/B_h).
    A single-unit bound does not hold: coarse ops whose kink lies inside
    their first unit make the literal greedy lose one partial unit per op."""
    rng = random.Random(12)
    for _ in range(1500):
        bg, bh = rng.uniform(2, 8), rng.uniform(0.2, 1.5)
        ops = _random_ops(rng, rng.randint(1, 4), dyadic=False)
        total = sum(o.bytes for o in ops)
        W = rng.randint(0, total)
        h = op.greedy_plan(ops, bg, bh, W)
        S = sum(hi * o.unit_bytes for hi, o in zip(h, ops))
        assert W <= S < W + max(o.unit_bytes for o in ops)
        best, _ = brute.best_plans(ops, bg, bh, W)
        gap = op.modeled_time(ops, h, bg, bh) - best
        units = sum(o.unit_bytes for o in ops) + max(o.unit_bytes for o in ops)
        assert -1e-12 <= gap <= units * (1 / bg + 1 / bh) + 1e-12


def _theorem_checks(ops, bg, bh, W, h):
    rng_ab = [op.argmin_range(o, bg, bh) for o in ops]
    mem = [op.memory_bound(o, bg, bh) for o in ops]
    A_mem = sum(a * o.unit_bytes for (a, _), o, m in zip(rng_ab, ops, mem) if m)
    B_all = sum(b * o.unit_bytes for (_, b), o in zip(rng_ab, ops))
    if W <= A_mem:           # Theorem 1: the budget goes to memory-bound ops only
        assert all(hi == 0 for hi, m in zip(h, mem) if not m)
        assert all(hi <= a for hi, (a, _), m in zip(h, rng_ab, mem) if m)
    elif W <= B_all:         # Theorem 2: memory-bound ops at their peak, none past the turning point
        assert all(hi >= a for hi, (a, _), m in zip(h, rng_ab, mem) if m)
        assert all(hi <= b for hi, (_, b) in zip(h, rng_ab))
    else:                    # Theorem 3: every op at least at its turning point
        assert all(hi >= b for hi, (_, b) in zip(h, rng_ab))


def test_theorem_invariants_hold_on_random_plans():
    rng = random.Random(13)
    for _ in range(600):
        bg, bh = rng.uniform(2, 8), rng.uniform(0.2, 1.5)
        ops = [op.Op(rng.randint(1, 40), rng.randint(1, 64), rng.random() * 30) for _ in range(rng.randint(1, 12))]
        total = sum(o.bytes for o in ops)
        W = rng.randint(0, total)
        _theorem_checks(ops, bg, bh, W, op.greedy_plan(ops, bg, bh, W))


def test_infeasible_and_empty_budgets():
    ops = [op.Op(4, 10, 0.0), op.Op(2, 7, 1.0)]
    with pytest.raises(op.Infeasible):
        op.greedy_plan(ops, 4.0, 1.0, 55)
    assert op.greedy_plan(ops, 4.0, 1.0, 54) == [4, 2]
    assert op.greedy_plan(ops, 4.0, 1.0, 0) == [0, 0]


def _continuous_optimum(ops, bg, bh, W):
    # Per-byte marginal cost is -1/B_g on each op's decreasing region, 0 on its
    # flat region, +1/B_h beyond its turning point; fill them in that order.
    t0 = sum(max(o.t_comp, o.bytes / bg) for o in ops)
    P1 = sum(cm.decreasing_end(o.bytes, o.t_comp, bg, bh) * o.bytes for o in ops)
    P2 = sum((cm.turning_point(o.bytes, o.t_comp, bg, bh)
              - cm.decreasing_end(o.bytes, o.t_comp, bg, bh)) * o.bytes for o in ops)
    return t0 - min(W, P1) / bg + max(0.0, W - P1 - P2) / bh


def test_fine_units_converge_to_continuous_optimum():
    rng = random.Random(14)
    bg, bh = 6.4e12, 5.75e10
    for _ in range(30):
        ops = []
        for _ in range(rng.randint(2, 8)):
            C = rng.randint(20, 400) * 2 ** 20
            n = rng.choice([64, 128, 256])
            u = C // n
            tc = rng.choice([0.0, rng.uniform(0.2, 3) * (n * u) / bg, rng.uniform(2, 50) * (n * u) / bg])
            ops.append(op.Op(n, u, tc))
        total = sum(o.bytes for o in ops)
        W = int(rng.uniform(0, 0.9) * total)
        h = op.greedy_plan(ops, bg, bh, W)
        t = op.modeled_time(ops, h, bg, bh)
        tol = 2 * len(ops) * max(o.unit_bytes for o in ops) * (1 / bg + 1 / bh)
        assert abs(t - _continuous_optimum(ops, bg, bh, W)) <= tol


def test_plan_spends_exactly_the_capacity_budget():
    ops = [op.Op(160, 1 << 20, 0.0), op.Op(16, 128 << 20, 0.0), op.Op(896, 1 << 20, 0.0)]
    h, t = op.plan(ops, 6.4e12, 5.75e10, 0.02)
    W = op.required_host_bytes(0.02, sum(o.bytes for o in ops))
    S = sum(hi * o.unit_bytes for hi, o in zip(h, ops))
    assert W <= S < W + max(o.unit_bytes for o in ops)
    assert t == op.modeled_time(ops, h, 6.4e12, 5.75e10)
    assert op.uniform_plan(ops, 0.25) == [40, 4, 224]
