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


def test_llama8b_attention_16x32768_full_size():
    # 16 requests x 32768 tokens, 32 query heads on 8 KV heads, hd 128, 25 % of
    # the requests' KV in pinned host memory.
    # Every (request, query head) row against the oracle.
    B, Hq, Hkv, D, ctx = 16, 32, 8, 128, 32768
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=0)
    scale = 1.0 / np.sqrt(D)
    out4 = run(q, K, V, 4, scale)
    ref = oa.decode_attention(to_f64(q), to_f64(K), to_f64(V), scale)
    worst = 0.0
    for b in range(B):
        for j in range(Hq):
            err = normwise_error(out4[b, j].numpy(), ref[b, j])
            worst = max(worst, err)
            assert err <= TOL, (b, j, err)
    print(f"16 x 32768 attention: worst per-row normwise error over all {B * Hq} rows {worst:.3e}")
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
    with pytest.raises(ValueError, match="ws holds"):        # the binding's size check
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, ws=small)
    # the library's own check of the byte count it is given
    import ctypes as C
    from tiered_memory_offloading_amd import _lib as L
    lib = dak.library()
    qd = q.cuda()
    out = torch.empty((2, 4, 128), dtype=torch.float32, device="cuda")
    d = kv.desc()
    st = lib.dak_splitk_decode_attn(qd.data_ptr(), C.byref(d), 4, C.c_float(0.1), out.data_ptr(), small.data_ptr(),
                                    16, None, None)
    assert st == L.DAK_EINVAL and b"workspace" in lib.dak_last_error()


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
    # every (request, query head) row against the oracle, one request at a time
    worst = 0.0
    for b in range(B):
        Kb, Vb = to_f64(K[b]), to_f64(V[b])
        qb = to_f64(q[b])
        for j in range(Hq):
            gk = oa.kv_group(j, Hq, Hkv)
            err = normwise_error(out4[b, j].numpy(), oa.attend_one(qb[j], Kb[gk], Vb[gk], scale))
            worst = max(worst, err)
            assert err <= TOL, (b, j, err)
    print(f"70B-shaped attention: worst per-row normwise error over all {B * Hq} rows {worst:.3e}")
    del K, V
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Host units of single KV heads, and ragged batches (per-request lengths)
# ---------------------------------------------------------------------------
def run_kv(q, K, V, h, scale, unit=dak.KV_UNIT_REQUEST, lens=None, cfg=None):
    kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=lens)
    out = dak.splitk_decode_attn(q.cuda(), kv, scale, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu()


def test_head_unit_splits_bit_identical():
    # Host shares in (request, KV head) steps: 8 units at batch 2 x 4 KV heads.
    B, Hq, Hkv, D, ctx = 2, 16, 4, 128, 3000
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=40)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention(to_f64(q), to_f64(K), to_f64(V), scale)
    base = run_kv(q, K, V, 0, scale)
    assert normwise_error(base.numpy(), ref) <= TOL
    for h in range(B * Hkv + 1):
        assert torch.equal(run_kv(q, K, V, h, scale, unit=dak.KV_UNIT_HEAD), base), h
    assert torch.equal(run_kv(q, K, V, 1, scale), base)


def test_ragged_lengths_match_the_oracle_at_every_split():
    # Lengths at the chunk edges (2048 tokens per chunk at this size) and a
    # single token.
    B, Hq, Hkv, D, ctx = 4, 8, 2, 128, 5000
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=41)
    lens = torch.tensor([5000, 1, 2049, 2048], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale, lens.tolist())
    base = run_kv(q, K, V, 0, scale, lens=lens)
    # per request: the one-token request's exact row would dominate a joint norm
    for b in range(B):
        err = normwise_error(base[b].numpy(), ref[b])
        print(f"ragged len {int(lens[b])} normwise error {err:.3e}")
        assert err <= TOL
    # and the lengths do matter: the full-length oracle is far from it
    full = oa.decode_attention(to_f64(q), to_f64(K), to_f64(V), scale)
    assert normwise_error(base[2].numpy(), full[2]) > 10 * TOL
    # request 1 has one valid position: its value row, exactly
    assert torch.equal(base[1], V[1, :, 0].float().repeat_interleave(Hq // Hkv, dim=0))
    for h in range(B + 1):
        assert torch.equal(run_kv(q, K, V, h, scale, lens=lens), base), h
    for h in (1, 3, 6):
        assert torch.equal(run_kv(q, K, V, h, scale, unit=dak.KV_UNIT_HEAD, lens=lens), base), h


def test_chunk_length_at_full_size_with_head_units_and_ragged_lengths():
    # 16 requests x 32768 tokens on 8 KV heads make 1024 work items of 4096
    # tokens: without a length array this launch takes 4096-token chunks, with
    # one (ragged batches) 2048-token chunks.  Head-unit host shares keep the
    # all-HBM bits in both, each tier's bytes are read once, and every valid
    # request's rows match the oracle.
    B, Hq, Hkv, D, ctx = 16, 32, 8, 128, 32768
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=43, device="cuda")
    ragged = torch.tensor([32768, 1, 4095, 4096, 4097, 8192, 2048, 2049, 30000, 12345, 16, 17, 20480, 4,
                           31000, 32767], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    for lens, chunks in ((None, 8), (ragged, 16)):
        kv = dak.place_kv(K, V, 0, ctx_lens=lens)
        assert dak.decode_attn_workspace_bytes(kv, Hq) == B * Hq * chunks * (D + 2) * 4
        del kv
        base = run_kv(q, K, V, 0, scale, lens=lens)
        n_of = [ctx] * B if lens is None else lens.tolist()
        for h, unit in ((3, dak.KV_UNIT_HEAD), (45, dak.KV_UNIT_HEAD), (2, dak.KV_UNIT_REQUEST)):
            kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=lens)
            out = dak.splitk_decode_attn(q, kv, scale, cfg=dak.LaunchConfig(byte_counters=cnt.zero_()))
            torch.cuda.synchronize()
            assert torch.equal(out.cpu(), base), (chunks, h, unit)
            per_unit = [n_of[u // Hkv] * D * 2 * 2 for u in range(B * Hkv)]
            hu = h if unit == dak.KV_UNIT_HEAD else h * Hkv
            assert cnt.tolist() == [sum(per_unit[:hu]), sum(per_unit[hu:])], (chunks, h, unit)
            del kv
        for b in (range(B) if lens is not None else (0, 7, 15)):
            n = n_of[b]
            Kb, Vb = to_f64(K[b, :, :n]), to_f64(V[b, :, :n])
            qb = to_f64(q[b])
            for j in range(Hq):
                gk = oa.kv_group(j, Hq, Hkv)
                err = normwise_error(base[b, j].numpy(), oa.attend_one(qb[j], Kb[gk], Vb[gk], scale))
                assert err <= TOL, (chunks, b, j, n, err)
    del K, V
    torch.cuda.empty_cache()


def test_ragged_kv_bytes_read_once():
    B, Hq, Hkv, D, ctx = 3, 4, 2, 128, 4100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=42)
    lens = torch.tensor([17, 4100, 2048], dtype=torch.int32)
    for unit, h, host_units in ((dak.KV_UNIT_REQUEST, 1, 2), (dak.KV_UNIT_HEAD, 3, 3)):
        kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=lens)
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, cfg=dak.LaunchConfig(byte_counters=cnt))
        torch.cuda.synchronize()
        per_unit = [int(lens[u // Hkv]) * D * 2 * 2 for u in range(B * Hkv)]
        assert cnt.tolist() == [sum(per_unit[:host_units]), sum(per_unit[host_units:])]


def test_ragged_and_unit_arguments_checked():
    B, Hq, Hkv, D, ctx = 2, 4, 2, 128, 64
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=43)
    kv = dak.place_kv(K, V, 1, ctx_lens=torch.tensor([64, 10]))
    kv.ctx_lens = torch.tensor([64, 10], dtype=torch.int32)   # host memory: refused
    with pytest.raises(dak.DakError):
        dak.splitk_decode_attn(q.cuda(), kv, 0.1)
    kv = dak.place_kv(K, V, 1)
    kv.unit = 7
    with pytest.raises(dak.DakError):
        dak.splitk_decode_attn(q.cuda(), kv, 0.1)


def test_ragged_lengths_clamped():
    # len <= 0: an empty softmax, NaN rows; len > ctx: read as ctx.
    B, Hq, Hkv, D, ctx = 3, 4, 2, 128, 700
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=44)
    full = run_kv(q, K, V, 1, 0.1)
    out = run_kv(q, K, V, 1, 0.1, lens=torch.tensor([0, -5, 10**6], dtype=torch.int32))
    assert torch.isnan(out[:2]).all()
    assert torch.equal(out[2], full[2])


def test_head_units_and_ragged_lengths_at_eight_grouped_heads():
    B, Hq, Hkv, D, ctx = 3, 64, 8, 128, 2100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=45)
    lens = torch.tensor([2100, 5, 1500], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale, lens.tolist())
    base = run_kv(q, K, V, 0, scale, lens=lens)
    for b in range(B):
        assert normwise_error(base[b].numpy(), ref[b]) <= TOL
    for h in (1, 7, 8, 13, 24):
        assert torch.equal(run_kv(q, K, V, h, scale, unit=dak.KV_UNIT_HEAD, lens=lens), base), h


def test_output_layout_checked_by_the_binding():
    q, K, V = synth.attn_inputs(2, 4, 1, 128, 64, seed=8)
    kv = dak.place_kv(K, V, 1)
    with pytest.raises(ValueError):
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, out=torch.empty((2, 4, 128), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, out=torch.empty((2, 128, 4), device="cuda").transpose(1, 2))


def test_eight_head_kv_bytes_read_once():
    # Eight grouped heads: one wave of a token half loads K, the other V.
    B, Hq, Hkv, D, ctx = 3, 16, 2, 128, 3100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=46)
    lens = torch.tensor([3100, 1030, 1], dtype=torch.int32)
    for unit, h in ((dak.KV_UNIT_REQUEST, 1), (dak.KV_UNIT_HEAD, 3)):
        kv = dak.place_kv(K, V, h, unit=unit, ctx_lens=lens)
        cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
        dak.splitk_decode_attn(q.cuda(), kv, 0.1, cfg=dak.LaunchConfig(byte_counters=cnt))
        torch.cuda.synchronize()
        per_unit = [int(lens[u // Hkv]) * D * 2 * 2 for u in range(B * Hkv)]
        hu = kv.host_units
        assert cnt.tolist() == [sum(per_unit[:hu]), sum(per_unit[hu:])]
