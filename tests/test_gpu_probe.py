"""Streaming-read probes on the GPU: plausible bandwidths for both tiers and
the concurrent (host + HBM) launch.  DAK paper §4.3.1, Fig. 7."""
import pytest
import torch

import tiered_memory_offloading_amd as dak

pytestmark = pytest.mark.gpu


def test_probes_report_plausible_bandwidths():
    assert torch.cuda.is_available()
    g = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    ms = dak.probe_read(g, 1024, 1, reps=3)
    bw_g = g.numel() / ms / 1e6
    ms = dak.probe_read(h, 16, 4, reps=3)
    bw_h = h.numel() / ms / 1e6
    print(f"HBM {bw_g:.0f} GB/s, host {bw_h:.1f} GB/s")
    assert 1000 < bw_g < 9000
    assert 5 < bw_h < 80
    t, mg, mh = dak.probe_read_concurrent(g, 1024, 4, h, 16, 4)
    print(f"concurrent: total {t:.3f} ms, hbm {mg:.3f} ms, host {mh:.3f} ms")
    assert 0 < mg <= t * 1.05 and 0 < mh <= t * 1.05


def test_probe_argument_errors():
    g = torch.empty(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(dak.DakError):
        dak.probe_read(g, 1, 3)
    with pytest.raises(dak.DakError):
        dak.probe_read(g, 0, 1)
    # the library sees allocations, not tensors: torch carves small tensors out
    # of larger segments, so overrun the whole segment
    with pytest.raises(dak.DakError):
        dak.probe_read(g, 1, 1, nbytes=1 << 30)
    cpu = torch.empty(4096, dtype=torch.uint8)   # pageable
    with pytest.raises(dak.DakError):
        dak.probe_read(cpu, 1, 1)


def test_allocations_of_4_gib_and_more_validate():
    # The range check must see the full size of large allocations (a 32-bit
    # size would make a 4 GiB buffer look empty and a 5 GiB one look 1 GiB).
    g = torch.empty((5 << 30) // 2, dtype=torch.bfloat16, device="cuda")
    ms = dak.probe_read(g, 1024, 1, reps=1, nbytes=(5 << 30) - 4096)
    assert ms > 0
    h = torch.empty((5 << 30) // 2, dtype=torch.bfloat16, pin_memory=True)
    ms = dak.probe_read(h, 16, 4, reps=1, nbytes=(5 << 30) - 4096)
    assert ms > 0
    del g, h


def test_mfma_probe_is_plausible():
    # 8 independent MFMA chains per wave on every SIMD: the rate must lie
    # between a third of MI355X's published dense bf16 peak (2.5 PFLOP/s) and
    # that peak, and scale with the work.
    ms1, tf1 = dak.probe_mfma(workgroups=1024, iters=2048, reps=3)
    ms2, tf2 = dak.probe_mfma(workgroups=1024, iters=4096, reps=3)
    print(f"MFMA probe {tf1:.0f} / {tf2:.0f} TFLOP/s")
    assert 800 < tf2 < 2600
    assert 1.6 < ms2 / ms1 < 2.4
