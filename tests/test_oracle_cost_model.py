"""Pins of the cost model (DAK paper §4.2.1, Fig. 6; walkthrough sections on the
offload-ratio model, the memory-bound peak and the compute-bound interval)."""
import json
import os

import numpy as np
import pytest

from oracle import cost_model as cm
from conftest import GOLDEN


def test_worked_example_balance_point():
    with open(os.path.join(GOLDEN, "turning_points.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        x = cm.memory_bound_peak_ratio(c["b_g"], c["b_h"])
        assert abs(100 * x - c["x_star_pct"]) <= c["abs_tol_pct"]


def test_memory_bound_peak_is_sum_of_bandwidths():
    C, bg, bh = 1e9, 4.0e12, 0.45e12
    xs = cm.memory_bound_peak_ratio(bg, bh)
    assert cm.t_gpu(C, xs, bg) == pytest.approx(cm.t_host(C, xs, bh), rel=1e-14)
    assert cm.effective_bandwidth(C, xs, 0.0, bg, bh) == pytest.approx(bg + bh, rel=1e-14)
    # strictly lower on both sides of the peak, rising then falling (Fig. 6 left)
    grid = np.linspace(0, 1, 201)
    eb = [cm.effective_bandwidth(C, x, 0.0, bg, bh) for x in grid]
    k = int(np.argmax(eb))
    assert abs(grid[k] - xs) <= 0.005
    assert all(eb[i] <= eb[i + 1] for i in range(k))
    assert all(eb[i] >= eb[i + 1] for i in range(k, 200))
    # beyond the peak EB follows the host link alone: B_h / x
    assert cm.effective_bandwidth(C, 0.5, 0.0, bg, bh) == pytest.approx(bh / 0.5, rel=1e-14)


def test_compute_bound_flat_then_host_bound():
    C, bg, bh = 1e9, 4.0e12, 0.5e12
    t_comp = 4 * C / bg                      # four times slower than reading HBM
    b_i = C / t_comp
    xs = cm.compute_bound_threshold(C, t_comp, bh)
    assert xs == pytest.approx(bh / b_i, rel=1e-15)
    assert not cm.is_memory_bound(C, t_comp, bg)
    for x in np.linspace(0, xs, 9):
        assert cm.effective_bandwidth(C, x, t_comp, bg, bh) == pytest.approx(b_i, rel=1e-14)
    assert cm.effective_bandwidth(C, xs * 1.5, t_comp, bg, bh) < b_i
    assert cm.turning_point(C, t_comp, bg, bh) == pytest.approx(xs, rel=1e-14)
    assert cm.decreasing_end(C, t_comp, bg, bh) == 0.0


def test_memory_bound_with_compute_floor_has_a_flat_bottom():
    # C/B_g > T_comp > C/(B_g+B_h): T falls to T_comp, stays, then rises.
    C, bg, bh = 1.0, 4.0, 1.0
    t_comp = 0.22                            # C/B_g = 0.25, C/(B_g+B_h) = 0.2
    assert cm.is_memory_bound(C, t_comp, bg)
    lo = cm.decreasing_end(C, t_comp, bg, bh)
    hi = cm.turning_point(C, t_comp, bg, bh)
    assert lo == pytest.approx(1 - t_comp * bg / C)
    assert hi == pytest.approx(bh * t_comp / C)
    assert lo < hi
    for x in np.linspace(lo, hi, 7):
        assert cm.op_time(C, x, t_comp, bg, bh) == pytest.approx(t_comp, rel=1e-12)
    assert cm.op_time(C, lo * 0.5, t_comp, bg, bh) > t_comp
    assert cm.op_time(C, min(1.0, hi * 1.5), t_comp, bg, bh) > t_comp


def test_turning_point_reduces_to_both_closed_forms():
    bg, bh = 8.0, 0.5
    C = 10.0
    assert cm.turning_point(C, 0.0, bg, bh) == pytest.approx(bh / (bh + bg))
    t_comp = 3.0
    assert cm.turning_point(C, t_comp, bg, bh) == pytest.approx(bh / (C / t_comp))
    assert cm.turning_point(C, 1e9, bg, bh) == 1.0


def test_unit_time_is_two_tier_roofline_for_memory_bound_ops():
    # With T_comp = 0 the modelled time is max((1-x)C/B_hbm, xC/B_host); dyadic
    # sizes and bandwidths make both sides exact.
    n, u, bg, bh = 16, 1 << 17, 2.0 ** 42, 2.0 ** 35
    C = n * u
    for h in range(n + 1):
        assert cm.unit_time(n, u, h, 0.0, bg, bh) == cm.two_tier_roofline_time(C, h / n, bg, bh)


def test_unit_time_matches_continuous_model_at_unit_boundaries():
    n, u, bg, bh, tc = 20, 1000, 3.0e12, 5.5e10, 1.1e-6
    for h in range(n + 1):
        assert cm.unit_time(n, u, h, tc, bg, bh) == pytest.approx(
            cm.op_time(n * u, h / n, tc, bg, bh), rel=1e-14)
