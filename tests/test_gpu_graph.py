"""HIP-graph capture of the split operators.

A decode step is replayed as a captured graph in serving (and `bench.py` times
its step that way).  The entry points allocate nothing and only launch kernels
on the caller's stream, so a captured step must reproduce the eager results
bit for bit, replay after replay, with eager work in between.  Every GEMM path
(FMA, staged, register MFMA, tiled), the FP8 GEMM, the dense attention and the
paged attention (ragged lengths, random pool pages) are captured, each with a
host share."""
import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_launches():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mats = []
    for M, K, N, h in [(320, 1000, 1, 2), (320, 1000, 16, 2), (512, 1024, 64, 3), (320, 1000, 100, 2),
                       (320, 1000, 300, 2), (512, 2048, 300, 3)]:   # the last splits K (a second kernel)
        A, X = synth.gemm_inputs(M, K, N, seed=M + N)
        mats.append((dak.place_matrix(A, 64, h), X.cuda(), torch.empty((N, M), dtype=torch.float32, device="cuda")))
    q, Kc, Vc = synth.attn_inputs(4, 8, 2, 128, 1000, seed=3)
    kv = dak.place_kv(Kc, Vc, 1)
    qd = q.cuda()
    out = torch.empty((4, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty((dak.decode_attn_workspace_bytes(kv, 8),), dtype=torch.uint8, device="cuda")
    scale = 128 ** -0.5
    f8 = []
    for M, K, N, h in [(320, 1024, 1, 2), (512, 1024, 64, 3)]:
        codes, rs, X = synth.fp8_gemm_inputs(M, K, N, seed=M + N + 1)
        f8.append((dak.place_matrix_fp8(codes, rs, 64, h), X.cuda(),
                   torch.empty((N, M), dtype=torch.float32, device="cuda")))
    lens = torch.tensor([1000, 17, 640, 333], dtype=torch.int32)
    pkv = dak.place_paged_kv(Kc, Vc, lens, 16, host_units=[1, 6], seed=4)
    pout = torch.empty((4, 8, 128), dtype=torch.float32, device="cuda")
    pws = torch.empty((dak.paged_decode_attn_workspace_bytes(pkv, 8),), dtype=torch.uint8, device="cuda")

    def step():
        for S, x, y in mats:
            dak.splitk_gemm(S, x, y=y)
        for S, x, y in f8:
            dak.splitk_gemm_fp8(S, x, y=y)
        dak.splitk_decode_attn(qd, kv, scale, out=out, ws=ws)
        dak.paged_decode_attn(qd, pkv, scale, out=pout, ws=pws)

    step()
    torch.cuda.synchronize()
    ref = [y.clone() for _, _, y in mats] + [y.clone() for _, _, y in f8] + [out.clone(), pout.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        step()
    torch.cuda.synchronize()

    outs = [y for _, _, y in mats] + [y for _, _, y in f8] + [out, pout]
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {rep}, output {i}"
        step()   # eager work between replays
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)
