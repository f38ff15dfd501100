"""Concurrent use of the library: three host threads drive the split GEMM, the
FP8 split GEMM and split decode attention on three streams at once, each with
a quarter of its data in host memory.  The entry points keep no device state
between calls and order their launches on the caller's stream, so every result
must equal the same call made alone, bit for bit."""
import threading

import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak

pytestmark = pytest.mark.gpu
ITERS = 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def test_three_threads_on_three_streams_match_solo_calls():
    M, K, m, N = 4096, 4096, 64, 16
    A, x = synth.gemm_inputs(M, K, N, seed=31, device="cuda")
    W = dak.place_matrix(A, m, (M // m) // 4)
    codes, scale, x8 = synth.fp8_gemm_inputs(M, K, N, seed=32, device="cuda")
    W8 = dak.place_matrix_fp8(codes, scale, m, (M // m) // 4)
    B, Hq, Hkv, D, ctx = 16, 32, 8, 128, 4096
    q, Kc, Vc = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=33, device="cuda")
    kv = dak.place_kv(Kc, Vc, B // 4)
    scale_attn = D ** -0.5
    x, x8, q = x.contiguous(), x8.contiguous(), q.contiguous()

    # Solo calls on the default stream.
    y_ref = dak.splitk_gemm(W, x)
    y8_ref = dak.splitk_gemm_fp8(W8, x8)
    o_ref = dak.splitk_decode_attn(q, kv, scale_attn)
    torch.cuda.synchronize()

    # Every output and workspace allocated up front; the threads only launch.
    ys = [torch.empty_like(y_ref) for _ in range(ITERS)]
    y8s = [torch.empty_like(y8_ref) for _ in range(ITERS)]
    os_ = [torch.empty_like(o_ref) for _ in range(ITERS)]
    ws = torch.empty(dak.decode_attn_workspace_bytes(kv, Hq), dtype=torch.uint8, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)]
    errors = []

    def run(k):
        try:
            s = streams[k]
            for i in range(ITERS):
                if k == 0:
                    dak.splitk_gemm(W, x, y=ys[i], stream=s)
                elif k == 1:
                    dak.splitk_gemm_fp8(W8, x8, y=y8s[i], stream=s)
                else:
                    dak.splitk_decode_attn(q, kv, scale_attn, out=os_[i], ws=ws, stream=s)
        except Exception as e:   # reported below, on the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=run, args=(k,)) for k in range(3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(ITERS):
        assert torch.equal(ys[i], y_ref), ("bf16 gemm", i)
        assert torch.equal(y8s[i], y8_ref), ("fp8 gemm", i)
        assert torch.equal(os_[i], o_ref), ("attention", i)
