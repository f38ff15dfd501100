"""GPU parity of the split decode attention against the fp64 oracle.
DAK paper §5: the KV cache is split along the batch; requests [0, h) in pinned
host memory.  Bars: normwise error <= 1e-2; bit-identical outputs for every h;
exact results in the special cases; KV bytes read once."""
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


def run(q, K, V, h, scale, cfg=None):
    kv = dak.place_kv(K, V, h)
    out = dak.splitk_decode_attn(q.cuda(), kv, scale, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("ctx", [1, 7, 16, 17, 255, 1024, 1025, 3000])
def test_small_shapes_all_splits(G, ctx):
    B, Hkv, D = 3, 2, 128
    q, K, V = synth.attn_inputs(B, Hkv * G, Hkv, D, ctx, seed=ctx + G)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention(to_f64(q), to_f64(K), to_f64(V), scale)
    outs = [run(q, K, V, h, scale) for h in range(B + 1)]
    err = normwise_error(outs[0].numpy(), ref)
    print(f"G={G} ctx={ctx} normwise error {err:.3e}")
    assert err <= TOL
    for h in range(1, B + 1):
        assert torch.equal(outs[h], outs[0]), f"h={h}"


def test_config3_full_size():
    # 16 requests x 32768 tokens, 32 query heads on 8 KV heads, hd 128, 25 % of
    # the requests' KV in pinned host memory.
    B, Hq, Hkv, D, ctx = 16, 32, 8, 128, 32768
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=0)
    scale = 1.0 / np.sqrt(D)
    out4 = run(q, K, V, 4, scale)
    g = torch.Generator().manual_seed(5)
    pairs = [(0, 0), (3, 31), (4, 0), (15, 31)] + [(int(b), int(j)) for b, j in
                                                   zip(torch.randint(0, B, (12,), generator=g),
                                                       torch.randint(0, Hq, (12,), generator=g))]
    for b, j in pairs:
        gk = oa.kv_group(j, Hq, Hkv)
        ref = oa.attend_one(to_f64(q[b, j]), to_f64(K[b, gk]), to_f64(V[b, gk]), scale)
        err = normwise_error(out4[b, j].numpy(), ref)
        assert err <= TOL, (b, j, err)
    for h in (0, 2, 8):
        assert torch.equal(run(q, K, V, h, scale), out4), h


def test_kv_bytes_read_once():
    B, Hq, Hkv, D, ctx = 4, 8, 2, 128, 2500
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=1)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    run(q, K, V, 1, 0.1, cfg=dak.LaunchConfig(byte_counters=cnt))
    per_req = 2 * Hkv * ctx * D * 2
    assert cnt.tolist() == [per_req * 1, per_req * 3]


def test_exact_special_cases():
    D = 128
    # ctx = 1: the single value row
    q, K, V = synth.attn_inputs(2, 4, 1, D, 1, seed=2)
    assert torch.equal(run(q, K, V, 1, 0.3), V[:, 0, 0][:, None, :].expand(2, 4, D).float())
    # equal keys and integer values with a power-of-two context: exact mean
    ctx = 2048
    K = torch.ones((2, 1, ctx, D), dtype=torch.bfloat16)
    V = synth.int_valued_bf16((2, 1, ctx, D), -2, 2, seed=3)
    q = torch.full((2, 2, D), 0.5, dtype=torch.bfloat16)
    mean = V.double().sum(dim=2) / ctx
    out = run(q, K, V, 1, 0.05)
    assert torch.equal(out.double(), mean.expand(2, 2, D))
    # constant V = 0.25: the output is 0.25 whatever the scores
    q, K, _ = synth.attn_inputs(2, 8, 2, D, 1500, seed=4)
    V = torch.full_like(K, 0.25)
    assert torch.equal(run(q, K, V, 1, 1.0 / np.sqrt(D)), torch.full((2, 8, D), 0.25))
    # a dominant key selects its value row
    ctx = 700
    K = torch.zeros((1, 1, ctx, D), dtype=torch.bfloat16)
    K[0, 0, 333, 0] = 64.0
    q = torch.zeros((1, 1, D), dtype=torch.bfloat16)
    q[0, 0, 0] = 64.0
    V = synth.attn_inputs(1, 1, 1, D, ctx, seed=5)[2]
    assert torch.equal(run(q, K, V, 0, 1.0)[0, 0], V[0, 0, 333].float())


def test_grouped_heads_read_their_kv_head():
    B, Hq, Hkv, D, ctx = 2, 16, 4, 128, 300
    q, K, _ = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=6)
    # KV head g holds V == 2^g (powers of two keep the weighted mean exact)
    V = torch.stack([torch.full((ctx, D), float(2 ** g)) for g in range(Hkv)])[None].expand(B, -1, -1, -1)
    V = V.to(torch.bfloat16).contiguous()
    out = run(q, K, V, 1, 0.1)
    for j in range(Hq):
        assert torch.all(out[:, j] == float(2 ** (j // 4)))


def test_attention_pointer_validation():
    q, K, V = synth.attn_inputs(2, 4, 1, 128, 64, seed=7)
    kv = dak.place_kv(K, V, 1)
    bad = dak.SplitKV(K[:1].clone(), kv.v_host, kv.k_hbm, kv.v_hbm, 2, 1, 1, 128, 64)
    with pytest.raises(dak.DakError):
        dak.splitk_decode_attn(q.cuda(), bad, 0.1)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dak.DakError):
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, ws=small)


def test_llama70b_attention_full_size():
    # 64 query heads on 8 KV heads (groups of 8), 16 requests x 32768 tokens,
    # generated on the GPU; sampled (request, head) pairs against the oracle and
    # bit-identity between 0 and 4 requests on the host.
    B, Hq, Hkv, D, ctx = 16, 64, 8, 128, 32768
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=9, device="cuda")
    scale = 1.0 / np.sqrt(D)
    out4 = run(q, K, V, 4, scale)
    out0 = run(q, K, V, 0, scale)
    assert torch.equal(out4, out0)
    for b, j in [(0, 0), (3, 63), (4, 7), (15, 8), (9, 40)]:
        gk = oa.kv_group(j, Hq, Hkv)
        ref = oa.attend_one(to_f64(q[b, j]), to_f64(K[b, gk]), to_f64(V[b, gk]), scale)
        assert normwise_error(out4[b, j].numpy(), ref) <= TOL, (b, j)
    del K, V
    torch.cuda.empty_cache()
