"""Pins of the host work-group count (DAK paper §4.1: wave alignment and a host
cap; walkthrough: waves = ceil(tiles / SMs))."""
from oracle import schedule as sc


def test_waves_formula():
    assert sc.waves(10, 4) == 3
    assert sc.waves(8, 4) == 2
    assert sc.waves(1, 16) == 1


def test_host_workgroups_examples():
    assert sc.host_workgroups(0, 16) == 0
    assert sc.host_workgroups(4, 16) == 4          # one wave, one group per item
    assert sc.host_workgroups(24, 16) == 12        # two full waves beat 16 + 8
    assert sc.host_workgroups(1024, 16) == 16
    assert sc.host_workgroups(100, 16) == 15       # 7 waves is the minimum under the cap


def test_host_workgroups_properties():
    for items in range(1, 200):
        for cap in (1, 3, 8, 16, 32):
            G = sc.host_workgroups(items, cap)
            assert 1 <= G <= min(cap, items)
            w = sc.waves(items, G)
            assert w == sc.waves(items, min(cap, items))     # no extra waves
            assert G == 1 or sc.waves(items, G - 1) > w       # no wasted groups


def test_strided_assignment_covers_each_item_once():
    for items in (0, 1, 7, 64):
        for G in (1, 3, 8):
            got = sorted(i for lst in sc.strided_items(items, G) for i in lst)
            assert got == list(range(items))
