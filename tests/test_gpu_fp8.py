"""GPU parity of the FP8-weight split GEMM against the fp64 oracle.

FP8 (OCP E4M3) weight codes with one fp32 scale per row, bf16 activations
(the pages run their models in FP8; DAK §4.1 splits the weight by
tile-rows).  Bars: normwise error <= 1e-2 (measured ~1e-7: products are exact,
only the fp32 sums round); bit-identical outputs for every host share; every
e4m3 code decoded as the format defines it; host bytes read once."""
import numpy as np
import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak
from oracle import fp8 as of
from oracle.gemm import normwise_error

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def run(codes, scale, x, m, h, cfg=None):
    S = dak.place_matrix_fp8(codes, scale, m, h)
    y = dak.splitk_gemm_fp8(S, x.cuda().contiguous(), cfg=cfg)
    torch.cuda.synchronize()
    return y.cpu()


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 9, 16, 17, 33, 64])
def test_every_code_and_split(N):
    # Every finite code, K not a multiple of 32 (a half step at the end).
    M, K, m = 192, 528, 64
    codes = synth.fp8_all_codes(M, K, seed=N)
    gen = torch.Generator().manual_seed(100 + N)
    scale = torch.rand(M, generator=gen) * 0.01 + 1e-3
    x = synth.gemm_inputs(16, K, N, seed=N)[1]
    ref = of.gemm_fp8(codes, scale, x)
    base = run(codes, scale, x, m, 0)
    err = normwise_error(base.numpy(), ref)
    print(f"N={N} normwise error {err:.3e}")
    assert err <= TOL
    for h in range(1, M // m + 1):
        assert torch.equal(run(codes, scale, x, m, h), base), h



def test_columns_do_not_depend_on_the_batch():
    # For 2 <= N <= 64 output column n is the same MFMA sequence on the same
    # activation row for any N > n: small batches stage fewer activation rows
    # (the others are recomputed from staged rows and dropped), which must not
    # change a bit.  N = 1 takes the FMA path (one fp32 FMA chain per lane,
    # then a fixed butterfly), whose sum order differs; it stays within the
    # oracle's bar of the same column.
    M, K, m = 256, 1040, 64
    codes = synth.fp8_all_codes(M, K, seed=3)
    scale = torch.rand(M, generator=torch.Generator().manual_seed(3)) * 0.01 + 1e-3
    x = synth.gemm_inputs(16, K, 64, seed=3)[1]
    for h in (0, 2):
        full = run(codes, scale, x, m, h)
        for N in (2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63):
            assert torch.equal(run(codes, scale, x[:N], m, h), full[:N]), (h, N)
        one = run(codes, scale, x[:1], m, h)
        assert normwise_error(one.numpy(), of.gemm_fp8(codes, scale, x[:1])) <= TOL

def test_power_of_two_scales_exact():
    # Integer-valued codes, power-of-two scales and integer activations: every
    # partial sum is an exact small integer, so the result is exact.
    ints = torch.tensor([0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0x00], dtype=torch.uint8)
    gen = torch.Generator().manual_seed(7)
    M, K = 128, 1024
    codes = ints[torch.randint(0, len(ints), (M, K), generator=gen)]
    scale = 2.0 ** torch.randint(-3, 3, (M,), generator=gen).float()
    x = torch.randint(-3, 4, (16, K), generator=gen).to(torch.bfloat16)
    ref = of.gemm_fp8(codes, scale, x)
    for h in (0, 1, 2):
        assert np.array_equal(run(codes, scale, x, 64, h).double().numpy(), ref)
        assert np.array_equal(run(codes, scale, x[:1], 64, h).double().numpy(), ref[:1])   # the FMA path


@pytest.mark.parametrize("name, M, K", [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)])
@pytest.mark.parametrize("N", [1, 16, 64])
def test_llama8b_linears_sampled(name, M, K, N):
    codes, scale, x = synth.fp8_gemm_inputs(M, K, N, seed=3, device="cuda")
    n = M // 64
    outs = [run(codes, scale, x, 64, h) for h in (0, n // 4, n)]
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])
    rows = torch.randperm(M, generator=torch.Generator().manual_seed(N))[:256].sort().values
    ref = of.gemm_fp8(codes.cpu()[rows], scale.cpu()[rows], x.cpu())
    err = normwise_error(outs[0][:, rows].numpy(), ref)
    print(f"{name} N={N} sampled normwise error {err:.3e}")
    assert err <= TOL


def test_host_bytes_read_once():
    M, K, m, h = 4096, 4096, 64, 16
    codes, scale, x = synth.fp8_gemm_inputs(M, K, 16, seed=4, device="cuda")
    for N in (16, 1):
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        run(codes, scale, x[:N], m, h, cfg=dak.LaunchConfig(byte_counters=cnt))
        assert cnt.tolist() == [h * m * K, (M - h * m) * K], N


@pytest.mark.parametrize("N", [1, 3])
def test_nan_code_poisons_its_row_only(N):
    M, K = 64, 256
    codes, scale, x = synth.fp8_gemm_inputs(M, K, N, seed=5)
    base = run(codes, scale, x, 64, 0)
    bad = codes.clone()
    bad[17, 100] = 0x7F
    y = run(bad, scale, x, 64, 1)
    assert torch.isnan(y[:, 17]).all()
    keep = [r for r in range(M) if r != 17]
    assert torch.equal(y[:, keep], base[:, keep])


def test_fp8_arguments_checked():
    codes, scale, x = synth.fp8_gemm_inputs(64, 256, 2049, seed=6)
    S = dak.place_matrix_fp8(codes, scale, 64, 0)
    with pytest.raises(dak.DakError) as e:
        dak.splitk_gemm_fp8(S, x.cuda())              # N = 2049
    assert e.value.status == -4   # DAK_EUNSUPPORTED
    with pytest.raises(dak.DakError) as e:            # a staged host part with N > 64
        dak.splitk_gemm_fp8(S, x[:65].cuda().contiguous(), cfg=dak.LaunchConfig(staged_host=True))
    assert e.value.status == -4
    S.row_scale = S.row_scale.cpu()                   # scales must be device memory
    with pytest.raises(dak.DakError):
        dak.splitk_gemm_fp8(S, x[:8].cuda().contiguous())
    codes2, scale2, x2 = synth.fp8_gemm_inputs(64, 264, 4, seed=7)   # K % 16 != 0
    S2 = dak.place_matrix_fp8(codes2, scale2, 64, 0)
    with pytest.raises(dak.DakError):
        dak.splitk_gemm_fp8(S2, x2.cuda())


@pytest.mark.parametrize("M, K, m, N", [(16, 16, 16, 1), (16, 16, 16, 64), (48, 32, 16, 7), (96, 4112, 32, 40)])
def test_small_and_ragged_shapes(M, K, m, N):
    # One 16-row item, a single half step of K, odd row counts per tile-row,
    # and K = 4096 + 16 (a chunk with one 16-wide piece).
    codes = synth.fp8_all_codes(M, K, seed=M + K)
    scale = torch.linspace(0.01, 0.02, M)
    x = synth.gemm_inputs(16, K, N, seed=N)[1]
    ref = of.gemm_fp8(codes, scale, x)
    base = run(codes, scale, x, m, 0)
    assert normwise_error(base.numpy(), ref) <= TOL
    for h in range(1, M // m + 1):
        assert torch.equal(run(codes, scale, x, m, h), base), h


# ---------------------------------------------------------------------------
# Wide activations (N > 64): the compute-bound tiled kernel with FP8 A tiles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N", [65, 257, 600])
@pytest.mark.parametrize("K", [528, 1056, 1024])
def test_wide_n_every_code_and_split(N, K):
    # Every finite code; M = 320 leaves a partial HBM tile and a partial host
    # block for every split; K = 528 ends in a half 32-k step, K = 1056 in a
    # half 64-k HBM step, K = 1024 in neither.
    M, m = 320, 64
    codes = synth.fp8_all_codes(M, K, seed=N + K)
    scale = torch.rand(M, generator=torch.Generator().manual_seed(N + K)) * 0.01 + 1e-3
    x = synth.gemm_inputs(16, K, N, seed=N + K)[1]
    ref = of.gemm_fp8(codes, scale, x)
    base = run(codes, scale, x, m, 0)
    err = normwise_error(base.numpy(), ref)
    print(f"N={N} K={K} normwise error {err:.3e}")
    assert err <= TOL
    for h in range(1, M // m + 1):
        assert torch.equal(run(codes, scale, x, m, h), base), h


def test_wide_n_power_of_two_scales_exact():
    ints = torch.tensor([0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0x00], dtype=torch.uint8)
    gen = torch.Generator().manual_seed(8)
    M, K, N = 512, 1024, 512
    codes = ints[torch.randint(0, len(ints), (M, K), generator=gen)]
    scale = 2.0 ** torch.randint(-3, 3, (M,), generator=gen).float()
    x = torch.randint(-3, 4, (N, K), generator=gen).to(torch.bfloat16)
    ref = of.gemm_fp8(codes, scale, x)
    for h in (0, 3, 8):
        assert np.array_equal(run(codes, scale, x, 64, h).double().numpy(), ref)


def test_wide_n_prefill_sampled():
    # The prefill-shaped GEMM (A 28672 x 8192, B 8192 x 2048) with FP8
    # weights: 256 sampled rows (all 2048 columns) against the oracle; the
    # all-HBM, a planner-sized and the all-host split bit-identical.
    M, K, N = 28672, 8192, 2048
    codes, scale, x = synth.fp8_gemm_inputs(M, K, N, seed=9, device="cuda")
    n = M // 64
    outs = [run(codes, scale, x, 64, h) for h in (0, 90, n)]
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])
    rows = torch.randperm(M, generator=torch.Generator().manual_seed(9))[:256].sort().values
    ref = of.gemm_fp8(codes.cpu()[rows], scale.cpu()[rows], x.cpu())
    err = normwise_error(outs[0][:, rows].numpy(), ref)
    print(f"prefill FP8 sampled normwise error {err:.3e}")
    assert err <= TOL


def test_wide_n_bytes_requested_per_column_tile():
    # Each A panel is requested once per 256-column tile of the output; host
    # panels by the work-groups of one host group, which share an XCD's L2.
    M, K, N, h = 1024, 1024, 512, 7
    codes, scale, x = synth.fp8_gemm_inputs(M, K, N, seed=10, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    run(codes, scale, x, 64, h, cfg=dak.LaunchConfig(byte_counters=cnt))
    assert cnt.tolist() == [2 * h * 64 * K, 2 * (M - h * 64) * K]


def test_wide_n_nan_code_poisons_its_row_only():
    M, K, N = 320, 512, 300
    codes, scale, x = synth.fp8_gemm_inputs(M, K, N, seed=11)
    base = run(codes, scale, x, 64, 0)
    bad = codes.clone()
    bad[17, 100] = 0x7F
    bad[300, 511] = 0xFF
    for h in (0, 1, 5):
        y = run(bad, scale, x, 64, h)
        assert torch.isnan(y[:, 17]).all() and torch.isnan(y[:, 300]).all()
        keep = [r for r in range(M) if r not in (17, 300)]
        assert torch.equal(y[:, keep], base[:, keep])


@pytest.mark.parametrize("M, K, N", [(512, 2048, 300), (64, 1024, 65), (512, 2080, 100)])
def test_wide_n_k_segments(M, K, N):
    # Shapes that split K (the FP8 tiled kernel starts at N > 64): every
    # code, all splits bit-identical, against the oracle; the row scale
    # multiplies the sum of the segments.
    assert dak.library().dak_splitk_gemm_fp8_workspace_bytes(M, K, N) > 0
    codes = synth.fp8_all_codes(M, K, seed=M + N)
    scale = torch.rand(M, generator=torch.Generator().manual_seed(M + N)) * 0.01 + 1e-3
    x = synth.gemm_inputs(16, K, N, seed=M + N)[1]
    ref = of.gemm_fp8(codes, scale, x)
    base = run(codes, scale, x, 64, 0)
    err = normwise_error(base.numpy(), ref)
    print(f"M={M} K={K} N={N} split normwise error {err:.3e}")
    assert err <= TOL
    for h in range(1, M // 64 + 1):
        assert torch.equal(run(codes, scale, x, 64, h), base), h
