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


@pytest.mark.parametrize("weights, kv_unit", [("bf16", dak.KV_UNIT_REQUEST), ("fp8", dak.KV_UNIT_HEAD)])
def test_planned_step_matches_the_oracle(weights, kv_unit):
    B, ctx = 4, 600
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
