"""The planned decode step (DAK §3 Overview: capacity bound, per-op planner,
placement, split kernels) on a small decoder, with bf16 or FP8 weights and
whole-request or (request, KV head) KV units.  A tight HBM budget forces host
units; the placed tensors themselves give the oracle's inputs."""
import numpy as np
import pytest
import torch

import tiered_memory_offloading_amd as dak
from oracle import attention as oa
from oracle import fp8 as of
from oracle.gemm import gemm, normwise_error, to_f64
from tiered_memory_offloading_amd.model import DecodeModel, DecoderShape

pytestmark = pytest.mark.gpu
TOL = 1e-2
SMALL = DecoderShape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024, layers=2)


def _cat(a, b):
    parts = [t.cpu() for t in (a, b) if t is not None and t.numel()]
    return torch.cat(parts, dim=0)


@pytest.mark.parametrize("weights, kv_unit, B", [("bf16", dak.KV_UNIT_REQUEST, 4), ("fp8", dak.KV_UNIT_HEAD, 4),
                                                  ("fp8", dak.KV_UNIT_REQUEST, 96)])
def test_planned_step_matches_the_oracle(weights, kv_unit, B):
    # B = 96: the linears run at N = 96, FP8 weights through the tiled kernel.
    ctx = 600
    probe = DecodeModel(SMALL, B, ctx, 6.4e12, 57.5e9, 1 << 40, weights=weights, kv_unit=kv_unit,
                        log=lambda *_: None)
    H = int(probe.footprint * 0.8)                        # x_global = 0.2
    del probe
    model = DecodeModel(SMALL, B, ctx, 6.4e12, 57.5e9, H, weights=weights, kv_unit=kv_unit, log=lambda *_: None)
    assert abs(model.x_global - 0.2) < 1e-6
    assert model.host_bytes >= model.x_global * model.footprint   # the capacity constraint holds
    assert sum(o.host_units for o in model.slots) > 0
    model.step()
    torch.cuda.synchronize()
    # the last op of each kind ran last with its own descriptor: check one GEMM and the attention
    for kind in ("down", "attn"):
        i = max(j for j, o in enumerate(model.slots) if o.kind == kind)
        o = model.slots[i]
        if kind == "attn":
            d = o.desc   # out holds the last layer's attention
            units = B * SMALL.n_kv_heads
            K = _cat(d.k_host, d.k_hbm).reshape(B, SMALL.n_kv_heads, ctx, SMALL.head_dim)
            V = _cat(d.v_host, d.v_hbm).reshape(B, SMALL.n_kv_heads, ctx, SMALL.head_dim)
            assert K.shape[0] * K.shape[1] == units
            ref = oa.decode_attention(to_f64(model.q), to_f64(K), to_f64(V), model.scale)
            assert normwise_error(model.out.cpu().numpy(), ref) <= TOL
        else:
            d = o.desc
            x = model.x[kind]
            if weights == "fp8":
                ref = of.gemm_fp8(_cat(d.host, d.hbm), d.row_scale, x)
            else:
                ref = gemm(to_f64(_cat(d.host, d.hbm)), to_f64(x))
            assert normwise_error(model.y[kind].cpu().numpy(), ref) <= TOL


LLAMA70B_TWO_LAYERS = DecoderShape(hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, layers=2)


@pytest.mark.parametrize("weights, kv_unit", [("bf16", dak.KV_UNIT_REQUEST), ("fp8", dak.KV_UNIT_HEAD)])
def test_70b_shaped_planned_layers_match_the_oracle(weights, kv_unit):
    # Two 70B-shaped layers (QKV 10240x8192, attention 64q/8kv over 16 x 32768
    # tokens, O 8192x8192, gate+up 57344x8192, down 8192x28672) at batch 16,
    # under an HBM budget of 97 % of the footprint (x_global = 0.03), so the
    # planner places host units.  Every op runs alone and is checked against
    # the oracle: 256 seeded rows of each GEMM (all 16 columns) and two
    # (request, KV head) pairs of each attention op (all 8 of their query
    # heads), with the oracle's inputs read back from the placed tiers.
    B, ctx = 16, 32768
    s = LLAMA70B_TWO_LAYERS
    kv_layer = 2 * B * s.n_kv_heads * ctx * s.head_dim * 2
    wbytes = (1 if weights == "fp8" else 2) * sum(M * K for _, M, K in s.linears())
    footprint = s.layers * (kv_layer + wbytes)
    H = int(footprint * 0.97)
    print(f"70B-shaped {weights} layers, kv unit {kv_unit}: footprint {footprint / 2**30:.2f} GiB, H {H / 2**30:.2f}",
          flush=True)
    model = DecodeModel(s, B, ctx, 6.4e12, 57.5e9, H, weights=weights, kv_unit=kv_unit, log=lambda *_: None)
    assert model.footprint == footprint
    assert model.host_bytes >= model.x_global * model.footprint
    kinds_with_host = {o.kind for o in model.slots if o.host_units}
    assert len(kinds_with_host) >= 2, kinds_with_host
    model.step()
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(70)
    G = s.n_q_heads // s.n_kv_heads
    worst = {}
    for i, o in enumerate(model.slots):
        model.run_op(i)
        torch.cuda.synchronize()
        if o.kind == "attn":
            out = model.out.cpu()
            q = to_f64(model.q)
            for _ in range(2):
                b = int(torch.randint(0, B, (1,), generator=g))
                kvh = int(torch.randint(0, s.n_kv_heads, (1,), generator=g))
                Kb, Vb = model.kv_block(i, b, kvh)
                Kf, Vf = to_f64(Kb), to_f64(Vb)
                for j in range(kvh * G, (kvh + 1) * G):
                    err = normwise_error(out[b, j].numpy(), oa.attend_one(q[b, j], Kf, Vf, model.scale))
                    worst["attn"] = max(worst.get("attn", 0.0), err)
        else:
            M = o.units * model.m
            rows = torch.randperm(M, generator=g)[:256].tolist()
            W, sc = model.weight_rows(i, rows)
            x = model.x[o.kind].cpu()
            ref = of.gemm_fp8(W, sc, x) if weights == "fp8" else gemm(to_f64(W), to_f64(x))
            err = normwise_error(model.y[o.kind].cpu()[:, rows].numpy(), ref)
            worst[o.kind] = max(worst.get(o.kind, 0.0), err)
    print(f"worst normwise error per kind: {worst}; host units per op: {[o.host_units for o in model.slots]}")
    assert set(worst) == {"qkv", "attn", "o", "gate_up", "down"}
    assert max(worst.values()) <= TOL
    del model
    torch.cuda.empty_cache()
