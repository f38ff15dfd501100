"""The copy-based prefetch baseline (DAK paper §2.3 and Fig. 2: host units
copied into an HBM staging buffer one op ahead, then read from HBM) runs the
same split kernels with the host part marked as a staged device copy.  Bars:
every output bit-identical to the direct split at the same placement, over
repeated back-to-back steps; within 1e-2 normwise of the fp64 oracle; the
flag refused where it is not built; the copy-interference probe reports a
read that overlapped the copy."""
import ctypes as C

import numpy as np
import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak
from tiered_memory_offloading_amd import _lib as L
from tiered_memory_offloading_amd.prefetch import PrefetchStep
from oracle import attention as oa
from oracle import fp8 as of
from oracle.gemm import gemm, normwise_error, to_f64

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dak.library()


def _ops():
    """A mixed sequence: GEMMs on every path the flag takes (N = 1, 16, 64,
    100; FP8 at N = 1 and 16), and split attention with request units and
    with ragged (request, KV head) units.  Each op writes its own output."""
    ops, refs, outs = [], [], []
    for seed, (M, K, N, h) in enumerate([(512, 1024, 1, 3), (1024, 768, 16, 5), (768, 512, 64, 2),
                                         (512, 512, 100, 4), (256, 256, 3, 0)]):
        A, X = synth.gemm_inputs(M, K, N, seed=80 + seed)
        S = dak.place_matrix(A, 64, h)
        x, y = X.cuda(), torch.empty((N, M), dtype=torch.float32, device="cuda")
        ops.append((S, lambda S_, cfg, x=x, y=y: dak.splitk_gemm(S_, x, y=y, cfg=cfg)))
        outs.append(y)
        refs.append(gemm(to_f64(A), to_f64(X)))
    for seed, N in enumerate((16, 1)):
        codes, scale, X = synth.fp8_gemm_inputs(512, 1024, N, seed=90 + seed)
        S8 = dak.place_matrix_fp8(codes, scale, 64, 3)
        x8, y8 = X.cuda(), torch.empty((N, 512), dtype=torch.float32, device="cuda")
        ops.append((S8, lambda S_, cfg, x8=x8, y8=y8: dak.splitk_gemm_fp8(S_, x8, y=y8, cfg=cfg)))
        outs.append(y8)
        refs.append(of.gemm_fp8(codes, scale, X))
    for seed, (B, Hq, Hkv, ctx, h, unit, lens) in enumerate([(4, 16, 4, 2500, 1, dak.KV_UNIT_REQUEST, None),
                                                              (3, 8, 2, 3000, 3, dak.KV_UNIT_HEAD, [3000, 17, 2049])]):
        q, K, V = synth.attn_inputs(B, Hq, Hkv, 128, ctx, seed=95 + seed)
        kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=None if lens is None else torch.tensor(lens))
        qd, o = q.cuda(), torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        scale_a = 1.0 / np.sqrt(128)
        ops.append((kv, lambda kv_, cfg, qd=qd, o=o, s=scale_a: dak.splitk_decode_attn(qd, kv_, s, out=o, cfg=cfg)))
        outs.append(o)
        refs.append(oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale_a, lens or [ctx] * B))
    return ops, refs, outs


def test_prefetched_step_is_bit_identical_to_the_direct_split():
    ops, refs, outs = _ops()
    for op, fn in ops:
        fn(op, None)
    torch.cuda.synchronize()
    direct = [o.cpu() for o in outs]
    for d, r in zip(direct, refs):
        assert normwise_error(d.numpy(), r) <= TOL
    pf = PrefetchStep(ops)
    assert pf.staging_bytes >= 2 * max(dak.prefetch.host_part_bytes(op) for op, _ in ops)
    for rep in range(3):     # back-to-back steps: the copies of one step overlap the end of the last
        for o in outs:
            o.fill_(float("nan"))
        pf.step()
        pf.step()
        torch.cuda.synchronize()
        for k, (o, d) in enumerate(zip(outs, direct)):
            assert torch.equal(o.cpu(), d), (rep, k)


def test_staged_launch_counts_every_byte_as_hbm():
    A, X = synth.gemm_inputs(512, 1024, 16, seed=97)
    S = dak.place_matrix(A, 64, 3)
    staged = torch.empty((3 * 64, 1024), dtype=torch.bfloat16, device="cuda")
    staged.copy_(S.host)
    Ss = dak.SplitMatrix(staged, S.hbm, 512, 1024, 64, 3)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    y = dak.splitk_gemm(Ss, X.cuda(), cfg=dak.LaunchConfig(byte_counters=cnt, staged_host=True))
    torch.cuda.synchronize()
    assert cnt.tolist() == [0, 512 * 1024 * 2]
    assert torch.equal(y.cpu(), dak.splitk_gemm(S, X.cuda()).cpu())


def test_staged_flag_refused_where_not_built():
    lib = dak.library()
    cfg = L.LaunchCfg(0, 0, L.DAK_FLAG_STAGED_HOST, 0, None)
    A, X = synth.gemm_inputs(256, 256, 300, seed=98)
    S = dak.place_matrix(A, 64, 1)
    staged = S.host.cuda()
    d = dak.SplitMatrix(staged, S.hbm, 256, 256, 64, 1).desc()
    y = torch.empty((300, 256), dtype=torch.float32, device="cuda")
    x = X.cuda()
    assert lib.dak_splitk_gemm(C.byref(d), x.data_ptr(), 300, y.data_ptr(), C.byref(cfg), None) == L.DAK_EUNSUPPORTED
    q, K, V = synth.attn_inputs(2, 4, 2, 128, 64, seed=99)
    pk = dak.place_paged_kv(K, V, [64, 64], 16, [1])
    with pytest.raises(dak.DakError) as e:
        dak.paged_decode_attn(q.cuda(), pk, 0.1, cfg=dak.LaunchConfig(staged_host=True))
    assert e.value.status == L.DAK_EUNSUPPORTED
    # without the flag a device buffer in the host slot is still refused
    with pytest.raises(dak.DakError):
        dak.splitk_gemm(dak.SplitMatrix(staged, S.hbm, 256, 256, 64, 1), x[:16].contiguous())


def test_copy_interference_probe_overlaps_reads_with_the_copy():
    from tiered_memory_offloading_amd.prefetch import concurrent_copy_stream
    hbm = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    side = concurrent_copy_stream()
    alone, beside, copy_ms, n = dak.probe_copy_interference(hbm, 1024, 1, src, dst, reps=16, copy_stream=side)
    print(f"1 GiB read alone {alone:.3f} ms, beside a 256 MiB copy {beside:.3f} ms ({n} reads overlapped); "
          f"copy {copy_ms:.2f} ms = {src.numel() / copy_ms / 1e6:.1f} GB/s")
    assert n >= 1
    assert 0.9 * alone <= beside <= 3.0 * alone
    assert 10.0 <= src.numel() / copy_ms / 1e6 <= 80.0
    with pytest.raises(dak.DakError):
        dak.probe_copy_interference(hbm, 1024, 1, src, dst, copy_stream=torch.cuda.current_stream())
