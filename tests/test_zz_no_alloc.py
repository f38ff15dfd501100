"""The allocation-free split decode attention (dak_splitk_decode_attn_noalloc,
for callers that cannot allocate device memory) against the entry point that
takes a caller workspace: the same bits, on two calls in a row whose second
is smaller, and within the oracle's bar of the fp64 oracle.  It passes alone
in a fresh process and after the other GPU tests (it is collected last)."""
import numpy as np
import pytest
import torch

import synth
import tiered_memory_offloading_amd as dak
from oracle import attention as oa
from oracle.gemm import to_f64, normwise_error

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dak.library()


def _case(B, Hq, Hkv, ctx, h, unit, lens, seed, stream=None):
    q, K, V = synth.attn_inputs(B, Hq, Hkv, 128, ctx, seed=seed)
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=lens_t)
    qd = q.cuda()
    scale = 1.0 / np.sqrt(128)
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        ref_out = dak.splitk_decode_attn(qd, kv, scale)
        out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        dak.splitk_decode_attn_noalloc(qd, kv, scale, out)
    torch.cuda.synchronize()
    return q, K, V, lens, scale, out.cpu(), ref_out.cpu()


def _check(q, K, V, lens, scale, out, ref_out):
    assert torch.equal(out, ref_out)
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale,
                                   lens if lens is not None else [K.shape[2]] * K.shape[0])
    for b in range(q.shape[0]):
        err = normwise_error(out[b].numpy(), ref[b])
        assert err <= TOL, (b, err)


def test_noalloc_matches_workspace_entry_point_on_two_calls_second_smaller():
    print("noalloc call 1: B=6 Hq=16 Hkv=4 ctx=5000 h=2 request units, ragged", flush=True)
    first = _case(6, 16, 4, 5000, 2, dak.KV_UNIT_REQUEST, [5000, 17, 2049, 4096, 1, 3333], seed=70)
    _check(*first)
    print("noalloc call 2: B=3 Hq=8 Hkv=2 ctx=1500 h=3 head units", flush=True)
    second = _case(3, 8, 2, 1500, 3, dak.KV_UNIT_HEAD, None, seed=71)
    _check(*second)


def test_noalloc_on_a_side_stream_and_at_the_largest_size_it_takes():
    # 16 requests x 32 query heads x 32768 tokens (4.3 MB of records) on a
    # stream of its own, then a small call after it on the default stream.
    side = torch.cuda.Stream()
    print("noalloc call: B=16 Hq=32 Hkv=8 ctx=32768 h=4 on a side stream", flush=True)
    q, K, V, lens, scale, out, ref_out = _case(16, 32, 8, 32768, 4, dak.KV_UNIT_REQUEST, None, seed=72,
                                               stream=side)
    assert torch.equal(out, ref_out)
    g = torch.Generator().manual_seed(9)
    for b, j in [(0, 0), (4, 31)] + [(int(b), int(j)) for b, j in zip(torch.randint(0, 16, (4,), generator=g),
                                                                        torch.randint(0, 32, (4,), generator=g))]:
        gk = oa.kv_group(j, 32, 8)
        ref = oa.attend_one(to_f64(q[b, j]), to_f64(K[b, gk]), to_f64(V[b, gk]), scale)
        assert normwise_error(out[b, j].numpy(), ref) <= TOL, (b, j)
    print("noalloc call: B=2 Hq=2 Hkv=2 ctx=40 h=1", flush=True)
    _check(*_case(2, 2, 2, 40, 1, dak.KV_UNIT_REQUEST, None, seed=73))
