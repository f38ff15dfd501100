"""Host-side rule of the drop-in modules: h = ceil(ratio * n) in exact
rationals (the same rounding as the oracle's host_units)."""
from fractions import Fraction

import pytest

from oracle.gemm import host_units as oracle_host_units
from tiered_memory_offloading_amd.nn import host_units


@pytest.mark.parametrize("ratio,n", [(0.0, 96), (0.1, 10), (0.25, 96), (0.05, 448), (1 / 3, 9), (0.3, 10),
                                     (Fraction(7, 20), 64), (1.0, 448), (0.999, 1000)])
def test_host_units_round_up_exactly(ratio, n):
    assert host_units(ratio, n) == oracle_host_units(ratio, n)


def test_host_units_reject_out_of_range():
    with pytest.raises(ValueError):
        host_units(-0.1, 10)
    with pytest.raises(ValueError):
        host_units(1.5, 10)
