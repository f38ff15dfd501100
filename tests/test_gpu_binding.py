"""The binding refuses buffers too small for the descriptors they go with,
before anything is launched, even when each view sits inside a larger
allocation (the library alone sees only the allocation that holds a pointer,
which under PyTorch's caching allocator is a whole pool segment).  And a
paged unit order that misses a unit gives NaN rows for it, not values an
earlier call left in the workspace."""
import numpy as np
import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dak.library()


def test_gemm_refuses_short_activations_and_weights():
    A, X = synth.gemm_inputs(256, 512, 4, seed=1)
    S = dak.place_matrix(A, 64, 1)
    big = torch.zeros((8, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="columns"):
        dak.splitk_gemm(S, big[:4, :256].contiguous())             # K of 256 against A's 512
    with pytest.raises(ValueError, match="columns"):
        dak.splitk_gemm(S, big.view(-1)[: 4 * 500].view(4, 500))   # a short view inside a larger block
    short = dak.SplitMatrix(S.host, S.hbm[:100], 256, 512, 64, 1)  # 100 of the 192 HBM rows
    with pytest.raises(ValueError, match="A.hbm"):
        dak.splitk_gemm(short, X.cuda())
    short = dak.SplitMatrix(S.host[:32], S.hbm, 256, 512, 64, 1)   # 32 of the 64 host rows
    with pytest.raises(ValueError, match="A.host"):
        dak.splitk_gemm(short, X.cuda())
    ok = dak.splitk_gemm(S, X.cuda())
    torch.cuda.synchronize()
    assert ok.shape == (4, 256)


def test_fp8_gemm_refuses_short_activations_and_scales():
    codes, scale, X = synth.fp8_gemm_inputs(128, 256, 2, seed=2)
    S = dak.place_matrix_fp8(codes, scale, 64, 1)
    with pytest.raises(ValueError, match="columns"):
        dak.splitk_gemm_fp8(S, torch.zeros((2, 128), dtype=torch.bfloat16, device="cuda"))
    short = dak.SplitMatrixFP8(S.host, S.hbm, S.row_scale[:64], 128, 256, 64, 1)
    with pytest.raises(ValueError, match="row_scale"):
        dak.splitk_gemm_fp8(short, X.cuda())


def test_attention_refuses_short_q_kv_and_workspace():
    B, Hq, Hkv, D, ctx = 4, 8, 2, 128, 300
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=3)
    kv = dak.place_kv(K, V, 1)
    qd = q.cuda()
    pool = torch.zeros((2 * B, Hq, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="q is"):
        dak.splitk_decode_attn(pool[: B - 1].contiguous(), kv, 0.1)   # one request short
    with pytest.raises(ValueError, match="q is"):
        dak.splitk_decode_attn(torch.zeros((B, Hq, 64), dtype=torch.bfloat16, device="cuda"), kv, 0.1)
    out_pool = torch.zeros((2 * B * Hq * D,), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="out"):
        dak.splitk_decode_attn(qd, kv, 0.1, out=out_pool[: (B - 1) * Hq * D].view(B - 1, Hq, D))
    need = dak.decode_attn_workspace_bytes(kv, Hq)
    ws_pool = torch.zeros((2 * need,), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="ws holds"):
        dak.splitk_decode_attn(qd, kv, 0.1, ws=ws_pool[: need - 4])
    short = dak.SplitKV(kv.k_host, kv.v_host, kv.k_hbm[:-1], kv.v_hbm, B, 1, Hkv, D, ctx)
    with pytest.raises(ValueError, match="k_hbm"):
        dak.splitk_decode_attn(qd, short, 0.1)
    short = dak.SplitKV(kv.k_host, kv.v_host[:1], kv.k_hbm, kv.v_hbm, B, 1, Hkv, D, ctx)
    with pytest.raises(ValueError, match="v_host"):
        dak.splitk_decode_attn(qd, short, 0.1)
    with pytest.raises(ValueError, match="q is"):
        dak.splitk_decode_attn_noalloc(pool[: B - 1].contiguous(), kv, 0.1,
                                       torch.empty((B - 1, Hq, D), dtype=torch.float32, device="cuda"))
    out = dak.splitk_decode_attn(qd, kv, 0.1)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_paged_attention_refuses_a_short_unit_order_and_page_table():
    B, Hq, Hkv, D, ctx = 2, 4, 2, 128, 100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=4)
    kv = dak.place_paged_kv(K, V, [100, 60], 16, [1])
    qd = q.cuda()
    bad = dak.PagedKV(kv.k_host, kv.v_host, kv.k_hbm, kv.v_hbm, kv.page_table, kv.ctx_lens, kv.unit_order[:3],
                      B, Hkv, D, 16, 1)
    with pytest.raises(ValueError, match="unit_order"):
        dak.paged_decode_attn(qd, bad, 0.1)
    bad = dak.PagedKV(kv.k_host, kv.v_host, kv.k_hbm, kv.v_hbm, kv.page_table[:3], kv.ctx_lens, kv.unit_order,
                      B, Hkv, D, 16, 1)
    with pytest.raises(ValueError, match="page_table"):
        dak.paged_decode_attn(qd, bad, 0.1)
    with pytest.raises(ValueError, match="q is"):
        dak.paged_decode_attn(qd[:1].contiguous(), kv, 0.1)


def test_paged_unit_order_that_misses_a_unit_gives_nan_rows_not_stale_ones():
    B, Hq, Hkv, D, ctx = 3, 8, 2, 128, 700
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=5)
    lens = [700, 300, 650]
    kv = dak.place_paged_kv(K, V, lens, 16, [0, 3], seed=1)
    qd = q.cuda()
    scale = 1.0 / np.sqrt(D)
    need = dak.paged_decode_attn_workspace_bytes(kv, Hq)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    good = dak.paged_decode_attn(qd, kv, scale, ws=ws).cpu()   # fills ws with valid records
    torch.cuda.synchronize()
    assert torch.isfinite(good).all()
    G = Hq // Hkv
    order = kv.unit_order.cpu().tolist()
    for name, corrupt in (("out of range", lambda o, i: 99), ("duplicate", lambda o, i: o[i - 1])):
        for i in (1, 4):    # a host slot and an HBM slot
            o = list(order)
            missed = o[i]
            o[i] = corrupt(o, i)
            bad = dak.PagedKV(kv.k_host, kv.v_host, kv.k_hbm, kv.v_hbm, kv.page_table, kv.ctx_lens,
                              torch.tensor(o, dtype=torch.int32, device="cuda"), B, Hkv, D, 16, kv.n_host_units)
            out = dak.paged_decode_attn(qd, bad, scale, ws=ws).cpu()
            torch.cuda.synchronize()
            b, g = divmod(missed, Hkv)
            rows = out[b, g * G:(g + 1) * G]
            assert torch.isnan(rows).all(), (name, i, missed)
            mask = torch.ones(B, Hq, dtype=torch.bool)
            mask[b, g * G:(g + 1) * G] = False
            assert torch.equal(out[mask], good[mask]), (name, i)
