"""GPU parity of the paged split decode attention.

Paged KV (BOOST §3.3, §4.3: pages of a few tokens from a free pool, reordered
head-major so single KV heads can live in the host tier), with DAK's rule that
every (request, KV head) attends within one tier.  Bars: normwise error <= 1e-2
against the fp64 oracle per request; bit-identical to the dense split kernel on
the same lengths, whatever the page size, the pool order or which units are
host units; KV bytes read once; bad page indices give NaN rows, never a read
outside a pool."""
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


def dense(q, K, V, lens, scale):
    kv = dak.place_kv(K, V, 0, ctx_lens=lens)
    out = dak.splitk_decode_attn(q.cuda(), kv, scale)
    torch.cuda.synchronize()
    return out.cpu()


def paged(q, K, V, lens, scale, page, host_units=(), seed=None, cfg=None):
    kv = dak.place_paged_kv(K, V, lens, page, host_units, seed=seed)
    out = dak.paged_decode_attn(q.cuda(), kv, scale, cfg=cfg)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("page", [16, 64, 2048, 4096])
def test_paged_matches_dense_and_oracle(page):
    B, Hq, Hkv, D, ctx = 3, 8, 2, 128, 4500
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=50)
    lens = torch.tensor([4500, 17, 2049], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale, lens.tolist())
    base = dense(q, K, V, lens, scale)
    out = paged(q, K, V, lens, scale, page)
    for b in range(B):
        err = normwise_error(out[b].numpy(), ref[b])
        print(f"page {page} request {b} len {int(lens[b])} normwise error {err:.3e}")
        assert err <= TOL
    assert torch.equal(out, base)
    # shuffled pools and any choice of host units: the same bits
    g = torch.Generator().manual_seed(page)
    for trial in range(3):
        hu = torch.randperm(B * Hkv, generator=g)[: trial * 2 + 1].tolist()
        assert torch.equal(paged(q, K, V, lens, scale, page, hu, seed=trial), base), (trial, hu)
    assert torch.equal(paged(q, K, V, lens, scale, page, range(B * Hkv), seed=7), base)


def test_single_head_host_requests():
    # BOOST's single-head-host block type: one KV head of some requests on the
    # host, the rest of the cache in HBM.
    B, Hq, Hkv, D, ctx = 4, 32, 8, 128, 2100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=51)
    lens = torch.tensor([2100, 1500, 64, 900], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    base = dense(q, K, V, lens, scale)
    hu = [0 * Hkv + 3, 2 * Hkv + 0]
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    out = paged(q, K, V, lens, scale, 16, hu, seed=1, cfg=dak.LaunchConfig(byte_counters=cnt))
    assert torch.equal(out, base)
    per_unit = [int(lens[u // Hkv]) * D * 2 * 2 for u in range(B * Hkv)]
    host = sum(per_unit[u] for u in hu)
    assert cnt.tolist() == [host, sum(per_unit) - host]


def test_bad_page_index_poisons_only_its_unit():
    B, Hq, Hkv, D, ctx = 2, 4, 2, 128, 3000
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=52)
    lens = torch.tensor([3000, 2500], dtype=torch.int32)
    base = dense(q, K, V, lens, 0.1)
    for host_units in ((), (1,), (0, 1, 2, 3)):
        kv = dak.place_paged_kv(K, V, lens, 16, host_units, seed=3)
        bad_unit = 1                                 # request 0, KV head 1: query heads 2, 3
        pool = kv.host_pages if bad_unit in host_units else kv.hbm_pages
        kv.page_table[bad_unit, 150] = pool          # one past the end of its pool
        out = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
        assert torch.isnan(out[0, 2:]).all()
        assert torch.equal(out[0, :2], base[0, :2]) and torch.equal(out[1], base[1])
        kv.page_table[bad_unit, 150] = -1
        out = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
        assert torch.isnan(out[0, 2:]).all() and torch.equal(out[1], base[1])


def test_host_units_without_a_host_pool_are_nan():
    B, Hq, Hkv, D, ctx = 2, 2, 2, 128, 100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=53)
    lens = torch.tensor([100, 100], dtype=torch.int32)
    kv = dak.place_paged_kv(K, V, lens, 16)
    base = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
    kv.n_host_units = 1                              # unit_order[0] = unit 0 read from an empty host pool
    out = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
    assert torch.isnan(out[0, 0]).all()
    assert torch.equal(out[0, 1], base[0, 1]) and torch.equal(out[1], base[1])


def test_unit_order_out_of_range_is_skipped():
    B, Hq, Hkv, D, ctx = 2, 2, 2, 128, 100
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=54)
    lens = torch.tensor([100, 60], dtype=torch.int32)
    kv = dak.place_paged_kv(K, V, lens, 32, (2,), seed=5)
    base = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
    assert kv.unit_order.tolist() == [2, 0, 1, 3]
    kv.unit_order[0] = -4                            # unit 2 (the host unit) is not computed
    kv.unit_order[1] = 1 << 30                       # nor unit 0
    out = dak.paged_decode_attn(q.cuda(), kv, 0.1).cpu()
    # units 1 and 3 (query head 1 of each request, G = 1) are unaffected
    assert torch.equal(out[0, 1], base[0, 1]) and torch.equal(out[1, 1], base[1, 1])
    # units 0 and 2, which no entry names any more, come out NaN
    assert torch.isnan(out[0, 0]).all() and torch.isnan(out[1, 0]).all()


def test_paged_arguments_checked():
    B, Hq, Hkv, D, ctx = 2, 4, 2, 128, 64
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=55)
    lens = torch.tensor([64, 10], dtype=torch.int32)
    for field, value in (("page", 48), ("page", 8), ("n_host_units", 5), ("n_host_units", -1)):
        kv = dak.place_paged_kv(K, V, lens, 16, (1,))
        setattr(kv, field, value)
        with pytest.raises((dak.DakError, ValueError)):   # the binding or the library refuses
            dak.paged_decode_attn(q.cuda(), kv, 0.1)
    kv = dak.place_paged_kv(K, V, lens, 16, (1,))
    kv.k_host = torch.zeros(kv.k_host.shape, dtype=torch.bfloat16)   # pageable host memory: refused
    assert not kv.k_host.is_pinned()
    with pytest.raises(dak.DakError):
        dak.paged_decode_attn(q.cuda(), kv, 0.1)
    kv = dak.place_paged_kv(K, V, lens, 16)
    kv.ctx_lens = kv.ctx_lens.cpu()                  # lengths must be device memory
    with pytest.raises(dak.DakError):
        dak.paged_decode_attn(q.cuda(), kv, 0.1)
    kv = dak.place_paged_kv(K, V, lens, 16)
    with pytest.raises((dak.DakError, ValueError)):
        dak.paged_decode_attn(q.cuda()[:, :3].contiguous(), kv, 0.1)   # 3 query heads over 2 KV heads


def test_eight_grouped_heads_and_largest_page():
    # The 70B grouping (64 query / 8 KV heads) and a page of 2^20 tokens
    # (every unit has one page, the chunk lies inside it).
    B, Hq, Hkv, D, ctx = 2, 64, 8, 128, 2200
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=56)
    lens = torch.tensor([2200, 700], dtype=torch.int32)
    scale = 1.0 / np.sqrt(D)
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), scale, lens.tolist())
    base = dense(q, K, V, lens, scale)
    for b in range(B):
        assert normwise_error(base[b].numpy(), ref[b]) <= TOL
    for page, hu in ((16, [3, 9, 12]), (1 << 20, [0, 15])):
        assert torch.equal(paged(q, K, V, lens, scale, page, hu, seed=page % 97), base), page
    kv = dak.place_paged_kv(K, V, lens, 1 << 20)
    assert kv.max_pages == 1
