"""Oracle of the host work-group count (DAK paper §4.1, "Kernel over Partitioned
Memory": host vs HBM SM counts follow the ratio, wave alignment and a congestion
cap; walkthrough: waves w = ceil(n_t / n_s); DAK §4.3.1: do not assign more host
SMs than needed).

Reading adopted: among G = 1..min(cap, items) host work-groups, take the one
with the fewest waves ceil(items / G); among those, the smallest G.
"""
from __future__ import annotations


def waves(items: int, groups: int) -> int:
    return -(-items // groups)


def host_workgroups(items: int, cap: int) -> int:
    if items <= 0:
        return 0
    if cap <= 0:
        raise ValueError("host work-group cap must be positive")
    best = None
    for G in range(1, min(cap, items) + 1):
        key = (waves(items, G), G)
        if best is None or key < best:
            best = key
    return best[1]


def strided_items(items: int, groups: int):
    """Static strided assignment: group g takes items g, g + G, g + 2G, ..."""
    return [list(range(g, items, groups)) for g in range(groups)]
